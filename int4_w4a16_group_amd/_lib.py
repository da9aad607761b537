"""ctypes binding of libw4moe.so: the ``w4_*`` C ABI under the same names.

Argument marshalling only.  Pointers may be given as ints or as objects with
``data_ptr()`` (torch tensors); ``stream`` is a HIP stream handle (int) or an
object with ``cuda_stream``; ``None`` means the null stream.  Non-zero
status codes raise :class:`W4Error`.  The library must have been built
(``int4_w4a16_group_amd.build``); nothing here falls back to another
implementation.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4moe.so")

W4_OK, W4_E_INVALID, W4_E_NO_SLOT, W4_E_CONTEXT_CAP, W4_E_BAD_SLOT, W4_E_NOT_READY, W4_E_HIP, W4_E_UNSUPPORTED = \
    0, -1, -2, -3, -4, -5, -6, -7
W4_K_DENSE, W4_K_MOE_GATEUP, W4_K_MOE_DOWN, W4_K_ATTENTION, W4_K_ROUTER, W4_K_MOE = 1, 2, 3, 4, 5, 6
W4_OPT_FUSED_MOE = 1
(W4_T_QKV, W4_T_O, W4_T_ROUTER, W4_T_GATE, W4_T_UP, W4_T_DOWN, W4_T_EMBED, W4_T_LM_HEAD, W4_T_ATTN_NORM,
 W4_T_MOE_NORM, W4_T_FINAL_NORM) = range(11)


class w4_model_desc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "n_experts",
                                          "top_k", "moe_inter", "vocab", "group")] + [
        ("rms_eps", C.c_float), ("rope_theta", C.c_float)]


class W4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None
_vp, _i32, _sz = C.c_void_p, C.c_int32, C.c_size_t
_SIGS = {
    "w4_arena_bytes": (_sz, [C.POINTER(w4_model_desc), _i32, _i32]),
    "w4_bank_bytes": (_sz, [C.POINTER(w4_model_desc)]),
    "w4_workspace_bytes": (_sz, [C.POINTER(w4_model_desc), _i32, _i32]),
    "w4_create": (C.c_int, [C.POINTER(w4_model_desc), _i32, _i32, _vp, _vp, _vp, C.POINTER(_vp)]),
    "w4_destroy": (None, [_vp]),
    "w4_bank_load": (C.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "w4_slot_alloc": (C.c_int, [_vp, _i32, _i32, C.POINTER(_i32)]),
    "w4_slot_seed": (C.c_int, [_vp, _i32, _vp, _vp, _vp]),
    "w4_slot_release": (C.c_int, [_vp, _i32]),
    "w4_slot_position": (C.c_int, [_vp, _i32, C.POINTER(_i32)]),
    "w4_slots_advance": (C.c_int, [_vp, _i32, C.POINTER(_i32)]),
    "w4_slot_read_kv": (C.c_int, [_vp, _i32, _vp, _vp, _vp]),
    "w4_slot_set_sampling": (C.c_int, [_vp, _i32, C.c_uint64, C.c_float, _i32, C.c_float]),
    "w4_prefill_workspace_bytes": (_sz, [C.POINTER(w4_model_desc), _i32, _i32]),
    "w4_slot_prefill": (C.c_int, [_vp, _i32, _vp, _vp, _sz, _vp, _vp, _vp, _vp]),
    "w4_check_errors": (C.c_int, [_vp]),
    "w4_read_probe": (C.c_int, [_vp, _sz, _vp, _i32, _i32, _vp]),
    "w4_sync_probe": (C.c_int, [_i32, _i32, _i32, _vp, _sz, _vp]),
    "w4_set_option": (C.c_int, [_vp, _i32, _i32]),
    "w4_route_noalloc": (C.c_int, [_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "w4_decode_step": (C.c_int, [_vp, _i32, C.POINTER(_i32), _vp, _vp, _vp, _vp, _vp]),
    "w4_gemm": (C.c_int, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp]),
    "w4_route": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "w4_moe": (C.c_int, [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "w4_attn_decode": (C.c_int, [_vp, _i32, _i32, C.POINTER(_i32), _vp, _vp, _vp, _vp, _vp]),
    "w4_layer_step": (C.c_int, [_vp, _i32, _i32, C.POINTER(_i32), _vp, _vp, _vp]),
    "w4_status_string": (C.c_char_p, [_i32]),
    "w4_last_error": (C.c_char_p, [_vp]),
    "w4_last_step_counts": (C.c_int, [_vp, C.POINTER(_i32), C.POINTER(_i32)]),
    "w4_profile_begin": (C.c_int, [_vp, _i32]),
    "w4_profile_end": (C.c_int, [_vp, C.POINTER(C.c_double), C.POINTER(_i32)]),
}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run int4_w4a16_group_amd.build.build() first")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_names():
    return list(_SIGS)


def _p(x):
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _s(stream):
    if stream is None:
        return None
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def _i32arr(vals):
    vals = [int(v) for v in vals]
    return (_i32 * max(1, len(vals)))(*vals), len(vals)


def desc_of(d) -> w4_model_desc:
    """Build a w4_model_desc from any object with the same field names."""
    if isinstance(d, w4_model_desc):
        return d
    out = w4_model_desc()
    for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k", "moe_inter",
              "vocab", "group"):
        setattr(out, n, int(getattr(d, n)))
    out.rms_eps = float(d.rms_eps)
    out.rope_theta = float(d.rope_theta)
    return out


def _check(ctx, rc):
    if rc != W4_OK:
        msg = lib().w4_last_error(ctx).decode()
        raise W4Error(rc, f"{lib().w4_status_string(rc).decode()}: {msg}")
    return rc


# ------------------------------------------------------------------ C ABI, same names
def w4_arena_bytes(desc, max_streams: int, cap: int) -> int:
    d = desc_of(desc)
    return lib().w4_arena_bytes(C.byref(d), max_streams, cap)


def w4_bank_bytes(desc) -> int:
    d = desc_of(desc)
    return lib().w4_bank_bytes(C.byref(d))


def w4_workspace_bytes(desc, max_streams: int, cap: int) -> int:
    d = desc_of(desc)
    return lib().w4_workspace_bytes(C.byref(d), max_streams, cap)


def w4_create(desc, max_streams: int, cap: int, arena, bank, workspace):
    d = desc_of(desc)
    out = _vp()
    rc = lib().w4_create(C.byref(d), max_streams, cap, _p(arena), _p(bank), _p(workspace), C.byref(out))
    if rc != W4_OK:
        raise W4Error(rc, lib().w4_status_string(rc).decode())
    return out.value


def w4_destroy(ctx):
    lib().w4_destroy(ctx)


def w4_bank_load(ctx, layer: int, tensor: int, expert: int, packed, scales, stream=None):
    return _check(ctx, lib().w4_bank_load(ctx, layer, tensor, expert, _p(packed), _p(scales), _s(stream)))


def w4_slot_alloc(ctx, prompt_len: int, max_new_tokens: int) -> int:
    s = _i32()
    _check(ctx, lib().w4_slot_alloc(ctx, prompt_len, max_new_tokens, C.byref(s)))
    return s.value


def w4_slot_seed(ctx, slot: int, k, v, stream=None):
    return _check(ctx, lib().w4_slot_seed(ctx, slot, _p(k), _p(v), _s(stream)))


def w4_slot_release(ctx, slot: int):
    return _check(ctx, lib().w4_slot_release(ctx, slot))


def w4_slot_position(ctx, slot: int) -> int:
    p = _i32()
    _check(ctx, lib().w4_slot_position(ctx, slot, C.byref(p)))
    return p.value


def w4_slots_advance(ctx, slots):
    arr, n = _i32arr(slots)
    return _check(ctx, lib().w4_slots_advance(ctx, n, arr))


def w4_prefill_workspace_bytes(desc, max_prompt: int, cap: int) -> int:
    d = desc_of(desc)
    return lib().w4_prefill_workspace_bytes(C.byref(d), max_prompt, cap)


def w4_slot_prefill(ctx, slot: int, tokens, workspace, ws_bytes: int, logits=None, next_ids=None, route_ids=None,
                    stream=None):
    return _check(ctx, lib().w4_slot_prefill(ctx, slot, _p(tokens), _p(workspace), ws_bytes, _p(logits),
                                             _p(next_ids), _p(route_ids), _s(stream)))


def w4_slot_set_sampling(ctx, slot: int, seed: int, temperature: float, top_k: int, top_p: float):
    return _check(ctx, lib().w4_slot_set_sampling(ctx, slot, seed & (2**64 - 1), temperature, top_k, top_p))


def w4_slot_read_kv(ctx, slot: int, k, v, stream=None):
    return _check(ctx, lib().w4_slot_read_kv(ctx, slot, _p(k), _p(v), _s(stream)))


def w4_read_probe(src, nbytes: int, sink, grid: int, nontemporal: int = 0, stream=None):
    return _check(None, lib().w4_read_probe(_p(src), nbytes, _p(sink), grid, nontemporal, _s(stream)))


def w4_set_option(ctx, option: int, value: int):
    return _check(ctx, lib().w4_set_option(ctx, option, value))


def w4_sync_probe(mode: int, grid: int, n: int, scratch, nbytes: int, stream=None):
    return _check(None, lib().w4_sync_probe(mode, grid, n, _p(scratch), nbytes, _s(stream)))


def w4_route_noalloc(B: int, n_experts: int, top_k: int, logits, ids, w, counts=None, offsets=None,
                     pair_stream=None, pair_rank=None, stream=None):
    return _check(None, lib().w4_route_noalloc(B, n_experts, top_k, _p(logits), _p(ids), _p(w), _p(counts),
                                               _p(offsets), _p(pair_stream), _p(pair_rank), _s(stream)))


def w4_check_errors(ctx):
    return _check(ctx, lib().w4_check_errors(ctx))


def w4_decode_step(ctx, slots, tokens, logits, next_ids, route_ids=None, stream=None):
    arr, n = _i32arr(slots)
    return _check(ctx, lib().w4_decode_step(ctx, n, arr, _p(tokens), _p(logits), _p(next_ids), _p(route_ids),
                                            _s(stream)))


def w4_gemm(ctx, layer: int, tensor: int, expert: int, B: int, x, y, stream=None):
    return _check(ctx, lib().w4_gemm(ctx, layer, tensor, expert, B, _p(x), _p(y), _s(stream)))


def w4_route(ctx, B: int, logits, ids, w, counts=None, offsets=None, pair_stream=None, pair_rank=None, stream=None):
    return _check(ctx, lib().w4_route(ctx, B, _p(logits), _p(ids), _p(w), _p(counts), _p(offsets), _p(pair_stream),
                                      _p(pair_rank), _s(stream)))


def w4_moe(ctx, layer: int, B: int, x, router_logits, y, route_ids=None, stream=None):
    return _check(ctx, lib().w4_moe(ctx, layer, B, _p(x), _p(router_logits), _p(y), _p(route_ids), _s(stream)))


def w4_attn_decode(ctx, layer: int, slots, q, k_new, v_new, o, stream=None):
    arr, n = _i32arr(slots)
    return _check(ctx, lib().w4_attn_decode(ctx, layer, n, arr, _p(q), _p(k_new), _p(v_new), _p(o), _s(stream)))


def w4_layer_step(ctx, layer: int, slots, h, route_ids=None, stream=None):
    arr, n = _i32arr(slots)
    return _check(ctx, lib().w4_layer_step(ctx, layer, n, arr, _p(h), _p(route_ids), _s(stream)))


def w4_status_string(status: int) -> str:
    return lib().w4_status_string(status).decode()


def w4_last_error(ctx) -> str:
    return lib().w4_last_error(ctx).decode()


def w4_last_step_counts(ctx):
    a, b = _i32(), _i32()
    _check(ctx, lib().w4_last_step_counts(ctx, C.byref(a), C.byref(b)))
    return a.value, b.value


def w4_profile_begin(ctx, kernel: int):
    return _check(ctx, lib().w4_profile_begin(ctx, kernel))


def w4_profile_end(ctx):
    ms, n = C.c_double(), _i32()
    _check(ctx, lib().w4_profile_end(ctx, C.byref(ms), C.byref(n)))
    return ms.value, n.value
