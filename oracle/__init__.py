"""CPU oracle of the batched int4 MoE decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library shares no code with
it and never calls it.

``liborc.so`` (``w4oracle.c``) is the oracle proper: fp32 accumulation over
int4 group-dequantised weights with fp16 storage points, one stream at a time.
``ref64`` is an independent float64 NumPy brute force used to pin it.
This module only marshals NumPy arrays to the C functions.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")


class _Model(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "hidden", "n_q", "n_kv", "head_dim", "n_experts",
                                          "top_k", "inter", "vocab", "group")] + [
        ("rms_eps", C.c_float), ("rope_theta", C.c_double)] + [
        (n, C.POINTER(C.c_void_p)) for n in ("attn_norm", "qkv_p", "qkv_s", "o_p", "o_s", "moe_norm",
                                             "r_p", "r_s", "gate_p", "gate_s", "up_p", "up_s",
                                             "down_p", "down_s")] + [
        (n, C.c_void_p) for n in ("emb_p", "emb_s", "final_norm", "lm_p", "lm_s")]


class _Arena(C.Structure):
    _fields_ = [("n_slots", C.c_int32), ("cap", C.c_int32), ("k", C.c_void_p), ("v", C.c_void_p)]


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = C.CDLL(path)
        L.orc_h2f.restype = C.c_float
        L.orc_h2f.argtypes = [C.c_uint16]
        L.orc_f2h.restype = C.c_uint16
        L.orc_f2h.argtypes = [C.c_float]
        L.orc_h2f_array.argtypes = [_u16p, _f32p, C.c_int64]
        L.orc_f2h_array.argtypes = [_f32p, _u16p, C.c_int64]
        L.orc_code_at.restype = C.c_int
        L.orc_code_at.argtypes = [_u8p, C.c_int]
        L.orc_w4_gemm.argtypes = [C.c_int] * 4 + [_u16p, _u8p, _u16p, C.c_void_p, C.c_void_p]
        L.orc_rmsnorm.argtypes = [C.c_int, _u16p, _u16p, C.c_float, _u16p]
        L.orc_rope.argtypes = [C.c_int, C.c_int, C.c_int, C.c_double, _u16p, _u16p]
        L.orc_attention.argtypes = [C.c_int] * 4 + [_u16p, C.c_void_p, C.c_void_p, C.c_int64, _u16p]
        L.orc_topk_softmax.argtypes = [C.c_int, C.c_int, _f32p, _i32p, _f32p]
        L.orc_route_weights.argtypes = [C.c_int, _f32p, _i32p, _f32p]
        L.orc_bucket.argtypes = [C.c_int] * 3 + [_i32p] * 5
        L.orc_moe.argtypes = [C.POINTER(_Model), C.c_int, C.c_int, _u16p, _f32p, C.c_void_p, _u16p, C.c_void_p,
                              C.c_void_p]
        L.orc_layer_step.argtypes = [C.POINTER(_Model), C.POINTER(_Arena), C.c_int, C.c_int, _i32p, _i32p,
                                     _u16p, C.c_void_p, C.c_void_p, C.c_void_p]
        L.orc_embed.argtypes = [C.POINTER(_Model), C.c_int, _i32p, _u16p]
        L.orc_decode_step.argtypes = [C.POINTER(_Model), C.POINTER(_Arena), C.c_int, _i32p, _i32p, _i32p,
                                      C.c_void_p, C.c_void_p, _i32p, C.c_void_p, C.c_void_p]
        L.orc_prefill.argtypes = [C.POINTER(_Model), C.POINTER(_Arena), C.c_int, C.c_int, _i32p, C.c_void_p,
                                  _u16p, _i32p, C.c_void_p, C.c_void_p]
        L.orc_attn_step.argtypes = [C.POINTER(_Model), C.POINTER(_Arena), C.c_int, C.c_int, _i32p, _i32p,
                                    _u16p, _u16p, _u16p, _u16p]
        L.orc_splitmix.restype = C.c_uint64
        L.orc_splitmix.argtypes = [C.c_uint64, C.c_uint64]
        L.orc_draw.restype = C.c_float
        L.orc_draw.argtypes = [C.c_uint64, C.c_uint64]
        L.orc_sample.restype = C.c_int32
        L.orc_sample.argtypes = [C.c_int, _u16p, C.c_float, C.c_int, C.c_float, C.c_uint64, C.c_uint64]
        L.orc_threads.restype = C.c_int
        L.orc_set_threads.argtypes = [C.c_int]
        L.orc_init()
        _lib = L
    return _lib


def _c(a, dt):
    a = np.ascontiguousarray(a, dtype=dt)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def threads() -> int:
    return lib().orc_threads()


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


# ---------------------------------------------------------------- primitives
def h2f(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().orc_h2f_array(h.ravel(), out.ravel(), h.size)
    return out


def f2h(f: np.ndarray) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_f2h_array(f.ravel(), out.ravel(), f.size)
    return out


def code_at(packed_row: np.ndarray, k: int) -> int:
    return lib().orc_code_at(_c(packed_row, np.uint8), k)


def w4_gemm(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, group: int, out: str = "f16"):
    """y = x . dequant(W)^T.  x fp16 bits [B,K]; packed [N,K/2]; scales fp16 bits [N,K/g]."""
    x = _c(x, np.uint16)
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.uint16)
    B, K = x.shape
    N = packed.shape[0]
    assert packed.shape == (N, K // 2) and scales.shape == (N, K // group)
    if out == "f16":
        y = np.empty((B, N), np.uint16)
        lib().orc_w4_gemm(B, N, K, group, x, packed, scales, _ptr(y), None)
    else:
        y = np.empty((B, N), np.float32)
        lib().orc_w4_gemm(B, N, K, group, x, packed, scales, None, _ptr(y))
    return y


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    x = _c(x, np.uint16)
    out = np.empty_like(x)
    g = _c(gamma, np.uint16)
    for b in range(x.shape[0]):
        lib().orc_rmsnorm(x.shape[1], x[b], g, eps, out[b])
    return out


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """x fp16 bits [nh, D] -> rotated copy."""
    x = _c(x, np.uint16)
    out = np.empty_like(x)
    lib().orc_rope(x.shape[0], x.shape[1], int(pos), float(theta), x, out)
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q fp16 [Hq,D]; k, v fp16 [npos, Hkv, D] -> o fp16 [Hq, D]."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    Hq, D = q.shape
    npos, Hkv, _ = k.shape
    o = np.empty_like(q)
    lib().orc_attention(Hq, Hkv, D, npos, q, k.ctypes.data, v.ctypes.data, Hkv * D, o)
    return o


def topk_softmax(logits: np.ndarray, k: int):
    logits = _c(logits, np.float32)
    B, E = logits.shape
    ids = np.empty((B, k), np.int32)
    w = np.empty((B, k), np.float32)
    for b in range(B):
        lib().orc_topk_softmax(E, k, logits[b], ids[b], w[b])
    return ids, w


def route_weights(logits: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax weights of ranked selections: logits f32 [B,E], ids int32 [B,k] -> w f32 [B,k]."""
    logits = _c(logits, np.float32)
    ids = _c(ids, np.int32)
    B, k = ids.shape
    w = np.empty((B, k), np.float32)
    for b in range(B):
        lib().orc_route_weights(k, logits[b], ids[b], w[b])
    return w


def route_ok(ids, logits, tol) -> bool:
    """Whether ranked expert ids are a top-k of the logits up to the tolerance
    (the acceptance rule for a routing decision taken elsewhere before the
    oracle replays it): k distinct experts; every selected logit >= every
    unselected one - t, and each rank's logit >= the next rank's - t, with
    t = tol * max|logits|.  Where all gaps around the top k exceed t, only the
    exact top-k in rank order passes."""
    ids = [int(i) for i in np.asarray(ids).ravel()]
    lg = np.asarray(logits, dtype=np.float64)
    if len(set(ids)) != len(ids) or min(ids) < 0 or max(ids) >= len(lg):
        return False
    t = tol * np.max(np.abs(lg))
    sel = lg[ids]
    rest = np.delete(lg, ids)
    if rest.size and sel.min() < rest.max() - t:
        return False
    return bool(np.all(sel[:-1] >= sel[1:] - t))


def _force(force, shape):
    """Forced ranked expert ids (int32, C order) or None."""
    if force is None:
        return None
    f = _c(force, np.int32)
    assert f.shape == shape, (f.shape, shape)
    return f


def splitmix(seed: int, pos: int) -> int:
    """Output number pos of the SplitMix64 generator started at seed."""
    return int(lib().orc_splitmix(seed & (2**64 - 1), pos))


def draw(seed: int, pos: int) -> float:
    """The sampler's uniform draw in [0, 1) for (seed, position)."""
    return float(lib().orc_draw(seed & (2**64 - 1), pos))


def sample(logits: np.ndarray, temperature: float, top_k: int, top_p: float, seed: int, pos: int) -> int:
    """Next token from one fp16 logits row (bits [V]) by temperature / top-k / top-p sampling."""
    row = _c(logits, np.uint16)
    return int(lib().orc_sample(row.size, row, float(temperature), int(top_k), float(top_p),
                                seed & (2**64 - 1), int(pos)))


def bucket(ids: np.ndarray, E: int):
    ids = _c(ids, np.int32)
    B, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    ps = np.empty(B * k, np.int32)
    pr = np.empty(B * k, np.int32)
    lib().orc_bucket(B, k, E, ids, counts, offsets, ps, pr)
    return counts, offsets, ps, pr


# ---------------------------------------------------------------- model level
class Model:
    """Binds canonical NumPy weights (int4_w4a16_group_amd.inputs.ModelWeights layout)."""

    def __init__(self, mw):
        d = mw.desc
        self.desc = d
        self._keep = []
        L = d.n_layers

        def tab(arrs):
            arrs = [np.ascontiguousarray(a) for a in arrs]
            self._keep.extend(arrs)
            t = (C.c_void_p * L)(*[a.ctypes.data for a in arrs])
            self._keep.append(t)
            return C.cast(t, C.POINTER(C.c_void_p))

        ly = mw.layers
        m = _Model()
        m.n_layers, m.hidden, m.n_q, m.n_kv, m.head_dim = L, d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim
        m.n_experts, m.top_k, m.inter, m.vocab, m.group = d.n_experts, d.top_k, d.moe_inter, d.vocab, d.group
        m.rms_eps, m.rope_theta = d.rms_eps, d.rope_theta
        m.attn_norm = tab([x.attn_norm for x in ly])
        m.qkv_p, m.qkv_s = tab([x.qkv.packed for x in ly]), tab([x.qkv.scales for x in ly])
        m.o_p, m.o_s = tab([x.o.packed for x in ly]), tab([x.o.scales for x in ly])
        m.moe_norm = tab([x.moe_norm for x in ly])
        m.r_p, m.r_s = tab([x.router.packed for x in ly]), tab([x.router.scales for x in ly])
        m.gate_p, m.gate_s = tab([x.gate.packed for x in ly]), tab([x.gate.scales for x in ly])
        m.up_p, m.up_s = tab([x.up.packed for x in ly]), tab([x.up.scales for x in ly])
        m.down_p, m.down_s = tab([x.down.packed for x in ly]), tab([x.down.scales for x in ly])
        if mw.embed is not None:
            for name, a in (("emb_p", mw.embed.packed), ("emb_s", mw.embed.scales),
                            ("final_norm", mw.final_norm), ("lm_p", mw.lm_head.packed),
                            ("lm_s", mw.lm_head.scales)):
                a = np.ascontiguousarray(a)
                self._keep.append(a)
                setattr(m, name, a.ctypes.data)
        self.m = m


class Arena:
    """The oracle's own KV store: K and V each [L][slots][cap][Hkv][D] fp16."""

    def __init__(self, desc, n_slots: int, cap: int, fill: float | None = 0.0):
        shape = (desc.n_layers, n_slots, cap, desc.n_kv_heads, desc.head_dim)
        self.k = np.zeros(shape, np.uint16)
        self.v = np.zeros(shape, np.uint16)
        if fill is not None and fill != 0.0:
            bits = np.array([fill], np.float16).view(np.uint16)[0]
            self.k[...] = bits
            self.v[...] = bits
        self.a = _Arena(n_slots, cap, self.k.ctypes.data, self.v.ctypes.data)

    def seed(self, slot: int, k: np.ndarray, v: np.ndarray):
        """k, v canonical [L][prompt_len][Hkv][D]."""
        p = k.shape[1]
        self.k[:, slot, :p] = k
        self.v[:, slot, :p] = v


def moe(model: Model, layer: int, x: np.ndarray, logits: np.ndarray, force=None):
    """force: ranked expert ids [B, top_k] replacing the top-k of the logits (a replayed
    routing decision), or None."""
    x = _c(x, np.uint16)
    logits = _c(logits, np.float32)
    B = x.shape[0]
    d = model.desc
    f = _force(force, (B, d.top_k))
    y = np.empty_like(x)
    ids = np.empty((B, d.top_k), np.int32)
    w = np.empty((B, d.top_k), np.float32)
    lib().orc_moe(C.byref(model.m), layer, B, x, logits, _ptr(f), y, ids.ctypes.data, w.ctypes.data)
    return y, ids, w


def embed(model: Model, tokens) -> np.ndarray:
    """h fp16 bits [B][hidden]: the dequantised embedding rows of tokens (step O1)."""
    tokens = _c(tokens, np.int32)
    h = np.empty((len(tokens), model.desc.hidden), np.uint16)
    lib().orc_embed(C.byref(model.m), len(tokens), tokens, h)
    return h


def layer_step(model: Model, arena: Arena, layer: int, slots, positions, h: np.ndarray, force=None):
    """force: ranked expert ids [B, top_k] replacing the router's top-k, or None."""
    h = _c(h, np.uint16).copy()
    slots = _c(slots, np.int32)
    positions = _c(positions, np.int32)
    d = model.desc
    B = h.shape[0]
    f = _force(force, (B, d.top_k))
    ids = np.empty((B, d.top_k), np.int32)
    lg = np.empty((B, d.n_experts), np.float32)
    lib().orc_layer_step(C.byref(model.m), C.byref(arena.a), layer, B, slots, positions, h, _ptr(f),
                         ids.ctypes.data, lg.ctypes.data)
    return h, ids, lg


def decode_step(model: Model, arena: Arena, slots, positions, tokens, want_logits=True, want_router=False,
                force=None):
    """force: ranked expert ids [n_layers, B, top_k] replacing every layer's top-k, or None."""
    slots = _c(slots, np.int32)
    positions = _c(positions, np.int32)
    tokens = _c(tokens, np.int32)
    d = model.desc
    B = len(slots)
    f = _force(force, (d.n_layers, B, d.top_k))
    logits = np.empty((B, d.vocab), np.uint16) if want_logits else None
    nxt = np.empty(B, np.int32)
    ids = np.empty((d.n_layers, B, d.top_k), np.int32)
    rl = np.empty((d.n_layers, B, d.n_experts), np.float32) if want_router else None
    lib().orc_decode_step(C.byref(model.m), C.byref(arena.a), B, slots, positions, tokens, _ptr(f),
                          _ptr(logits), nxt, ids.ctypes.data, _ptr(rl))
    return logits, nxt, ids, rl


def prefill(model: Model, arena: Arena, slot: int, tokens, force=None, want_ids=False, want_router=False):
    """The prompt tokens through the model at positions 0..P-1 of the slot (its K/V
    written there); returns the last token's fp16 logits [V], its greedy id, and, if
    asked, the expert ids [n_layers, P, top_k] and the router logits [n_layers, P, E]
    (else None).  force: ranked expert ids [n_layers, P, top_k] replacing every top-k."""
    tokens = _c(tokens, np.int32)
    d = model.desc
    P = len(tokens)
    f = _force(force, (d.n_layers, P, d.top_k))
    logits = np.empty(d.vocab, np.uint16)
    nxt = np.empty(1, np.int32)
    ids = np.empty((d.n_layers, P, d.top_k), np.int32) if want_ids else None
    rl = np.empty((d.n_layers, P, d.n_experts), np.float32) if want_router else None
    lib().orc_prefill(C.byref(model.m), C.byref(arena.a), int(slot), P, tokens, _ptr(f), logits, nxt, _ptr(ids),
                      _ptr(rl))
    if want_router:
        return logits, int(nxt[0]), ids, rl
    return logits, int(nxt[0]), ids


def attn_step(model: Model, arena: Arena, layer: int, slots, positions, q, k_new, v_new):
    q = _c(q, np.uint16)
    o = np.empty_like(q)
    lib().orc_attn_step(C.byref(model.m), C.byref(arena.a), layer, len(slots), _c(slots, np.int32),
                        _c(positions, np.int32), q, _c(k_new, np.uint16), _c(v_new, np.uint16), o)
    return o
