"""Device-memory plumbing around the C ABI: torch allocates the arena, bank and
workspace; canonical host weights are copied to the device and handed to
``w4_bank_load``.  No arithmetic of the decode step happens here."""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L


def _dev(a: np.ndarray, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.to(device, non_blocking=False)


class Context:
    """Owns the device buffers of one w4_ctx.  ``desc`` is any object with the
    w4_model_desc field names (e.g. inputs.ModelDesc)."""

    def __init__(self, desc, max_streams: int, cap: int, device="cuda"):
        self.desc = desc
        self.max_streams, self.cap = max_streams, cap
        self.device = torch.device(device)
        self.arena_bytes = L.w4_arena_bytes(desc, max_streams, cap)
        self.bank_bytes = L.w4_bank_bytes(desc)
        self.ws_bytes = L.w4_workspace_bytes(desc, max_streams, cap)
        if not (self.arena_bytes and self.bank_bytes and self.ws_bytes):
            raise L.W4Error(L.W4_E_INVALID, "unsupported geometry")
        self.arena = torch.empty(self.arena_bytes, dtype=torch.uint8, device=self.device)
        self.bank = torch.empty(self.bank_bytes, dtype=torch.uint8, device=self.device)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.ctx = L.w4_create(desc, max_streams, cap, self.arena, self.bank, self.ws)

    def close(self):
        if self.ctx:
            torch.cuda.synchronize(self.device)
            L.w4_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def stream(self):
        return torch.cuda.current_stream(self.device)

    # ---- bank upload from canonical host arrays (inputs.ModelWeights layout)
    def load_tensor(self, layer: int, tensor: int, expert: int, packed: np.ndarray, scales: np.ndarray | None):
        p = _dev(packed, self.device)
        s = _dev(scales, self.device) if scales is not None else None
        L.w4_bank_load(self.ctx, layer, tensor, expert, p, s, self.stream)
        torch.cuda.current_stream(self.device).synchronize()   # sources may be freed after this

    def load_layer(self, l: int, lw):
        self.load_tensor(l, L.W4_T_ATTN_NORM, 0, lw.attn_norm, None)
        self.load_tensor(l, L.W4_T_MOE_NORM, 0, lw.moe_norm, None)
        self.load_tensor(l, L.W4_T_QKV, 0, lw.qkv.packed, lw.qkv.scales)
        self.load_tensor(l, L.W4_T_O, 0, lw.o.packed, lw.o.scales)
        self.load_tensor(l, L.W4_T_ROUTER, 0, lw.router.packed, lw.router.scales)
        self.load_tensor(l, L.W4_T_GATE, -1, lw.gate.packed, lw.gate.scales)
        self.load_tensor(l, L.W4_T_UP, -1, lw.up.packed, lw.up.scales)
        self.load_tensor(l, L.W4_T_DOWN, -1, lw.down.packed, lw.down.scales)

    def load_model(self, mw):
        for l, lw in enumerate(mw.layers):
            self.load_layer(l, lw)
        if mw.embed is not None:
            self.load_tensor(0, L.W4_T_EMBED, 0, mw.embed.packed, mw.embed.scales)
            self.load_tensor(0, L.W4_T_LM_HEAD, 0, mw.lm_head.packed, mw.lm_head.scales)
            self.load_tensor(0, L.W4_T_FINAL_NORM, 0, mw.final_norm, None)

    # ---- slots
    def join(self, prompt_len: int, max_new: int, k: np.ndarray | None = None, v: np.ndarray | None = None) -> int:
        s = L.w4_slot_alloc(self.ctx, prompt_len, max_new)
        if prompt_len > 0:
            kd, vd = _dev(k, self.device), _dev(v, self.device)
            L.w4_slot_seed(self.ctx, s, kd, vd, self.stream)
            torch.cuda.current_stream(self.device).synchronize()
        return s

    def prefill(self, tokens, max_new: int, logits=None, next_ids=None, route_ids=None) -> int:
        """A new stream whose prompt token ids go through the model (seed-at-join
        prefill); returns its slot.  tokens: host ints or a device int32 tensor."""
        t = tokens if isinstance(tokens, torch.Tensor) else torch.tensor(np.asarray(tokens, np.int32))
        t = t.to(self.device, dtype=torch.int32)
        P = int(t.numel())
        nbytes = L.w4_prefill_workspace_bytes(self.desc, P, self.cap)
        if not nbytes:
            raise L.W4Error(L.W4_E_UNSUPPORTED, "prompt too long for the prefill")
        if getattr(self, "_pf_ws", None) is None or self._pf_ws.numel() < nbytes:
            self._pf_ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        s = L.w4_slot_alloc(self.ctx, P, max_new)
        try:
            L.w4_slot_prefill(self.ctx, s, t, self._pf_ws, self._pf_ws.numel(), logits, next_ids, route_ids,
                              self.stream)
        except Exception:
            L.w4_slot_release(self.ctx, s)
            raise
        return s

    def release(self, slot: int):
        L.w4_slot_release(self.ctx, slot)

    def position(self, slot: int) -> int:
        return L.w4_slot_position(self.ctx, slot)

    def read_kv(self, slot: int):
        """The K/V a slot holds at positions 0..p-1 as host arrays, canonical
        [n_layers][p][n_kv][head_dim] fp16 bits (the inverse of seeding)."""
        d = self.desc
        p = self.position(slot)
        shape = (d.n_layers, p, d.n_kv_heads, d.head_dim)
        k = torch.empty(shape, dtype=torch.int16, device=self.device)
        v = torch.empty(shape, dtype=torch.int16, device=self.device)
        L.w4_slot_read_kv(self.ctx, slot, k, v, self.stream)
        torch.cuda.current_stream(self.device).synchronize()
        return k.cpu().numpy().view(np.uint16), v.cpu().numpy().view(np.uint16)
