"""Seeded synthetic inputs for the batched int4 MoE decode step.

This module draws numbers and lays them out in the canonical formats that
both the CPU oracle and the GPU library take as *data*.  It holds none of
the method's arithmetic: no dequantisation, no products, no norms, no
routing.  Its only encodings are the storage formats themselves:

* int4 weights ``W[N][K]``: byte ``P[n][j]`` holds element ``2j`` in bits
  0-3 and element ``2j+1`` in bits 4-7, each a 4-bit two's-complement code
  in [-8, 7].  Uniform codes are produced by drawing uniform random bytes,
  since every nibble of a uniform byte is a uniform 4-bit code.
* scales ``S[N][K/g]`` fp16 (IEEE binary16, round-to-nearest-even from a
  float64 draw), stored as ``uint16`` bit patterns.
* activations and KV values fp16 bit patterns, likewise.

Random bytes for weight banks come from the SplitMix64 counter-based
generator (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; constants as in Vigna's public-domain
``splitmix64.c``), so any tensor, or any row range of one, regenerates
independently and in parallel.  Everything else comes from NumPy's PCG64
with per-tensor child seeds ``[seed, tag, ...]``.

Workload shapes follow the five configurations of the int4 MoE decode
study ("Batched-concurrent 4-bit serving on Apple Silicon", section 3:
a 30B-class 4-bit MoE decoded by B concurrent greedy streams; "Per-stream
KV-slot isolation ...", section 1: streams join and finish at any step,
each in a stable KV slot).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_S30, _S27, _S31 = np.uint64(30), np.uint64(27), np.uint64(31)

# tensor tags for child seeds / SplitMix keys
T_QKV, T_O, T_ROUTER, T_GATE, T_UP, T_DOWN, T_EMBED, T_LM = range(1, 9)
T_QKV_S, T_O_S, T_ROUTER_S, T_GATE_S, T_UP_S, T_DOWN_S, T_EMBED_S, T_LM_S = range(11, 19)
T_X, T_LOGITS, T_KV, T_Q, T_KNEW, T_VNEW, T_SCHED, T_TOKENS, T_PERM = range(21, 30)


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------
def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function, in place on a uint64 array."""
    z ^= z >> _S30
    z *= _M1
    z ^= z >> _S27
    z *= _M2
    z ^= z >> _S31
    return z


def splitmix_key(*ids: int) -> int:
    """Fold integer ids into one 64-bit stream key."""
    k = np.array([0x243F6A8885A308D3], dtype=np.uint64)
    with np.errstate(over="ignore"):
        for i in ids:
            k = k + np.uint64(int(i) & 0xFFFFFFFFFFFFFFFF) * _GOLDEN + _GOLDEN
            k = _mix64(k)
    return int(k[0])


def splitmix_bytes(key: int, nbytes: int, start: int = 0, out: np.ndarray | None = None,
                   threads: int | None = None, lut: np.ndarray | None = None) -> np.ndarray:
    """Bytes ``start .. start+nbytes`` of the SplitMix64 stream for ``key``.

    Output word i is mix(key + (i+1)*golden); its 8 little-endian bytes are
    stream bytes 8i..8i+7.  ``start`` must be a multiple of 8.  ``lut`` (256
    bytes) optionally maps every byte afterwards.
    """
    assert start % 8 == 0
    if out is None:
        out = np.empty(nbytes, dtype=np.uint8)
    nwords = (nbytes + 7) // 8
    w0 = start // 8
    chunk = 1 << 20
    kk = np.uint64(key)

    def job(c0: int) -> None:
        c1 = min(c0 + chunk, nwords)
        with np.errstate(over="ignore"):
            z = (np.arange(w0 + c0 + 1, w0 + c1 + 1, dtype=np.uint64) * _GOLDEN) + kk
            _mix64(z)
        b = z.view(np.uint8)
        lo = c0 * 8
        hi = min(c1 * 8, nbytes)
        out[lo:hi] = b[: hi - lo] if lut is None else lut[b[: hi - lo]]

    starts = range(0, nwords, chunk)
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if nwords > chunk and threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(job, starts))
    else:
        for c0 in starts:
            job(c0)
    return out


def rng(*ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(i) for i in ids]))


def f16_bits(a: np.ndarray) -> np.ndarray:
    """float64/float32 array -> fp16 bit patterns (round to nearest even)."""
    return np.ascontiguousarray(a).astype(np.float16).view(np.uint16)


def normal_f16(g: np.random.Generator, shape) -> np.ndarray:
    return f16_bits(g.standard_normal(shape, dtype=np.float64))


def uniform_f16(g: np.random.Generator, lo: float, hi: float, shape) -> np.ndarray:
    return f16_bits(g.uniform(lo, hi, shape))


# --------------------------------------------------------------------------
# model description and weight sets
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class ModelDesc:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_experts: int
    top_k: int
    moe_inter: int
    vocab: int
    group: int
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0

    @property
    def n_qkv(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim


# tiny single MoE decoder layer (parity case)
TINY = ModelDesc(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                 n_experts=8, top_k=2, moe_inter=128, vocab=64, group=32)
# 30B-class MoE (48 layers, 128 experts top-8, vocab 151936, group 128)
FULL = ModelDesc(n_layers=48, hidden=2048, n_q_heads=32, n_kv_heads=4, head_dim=128,
                 n_experts=128, top_k=8, moe_inter=768, vocab=151936, group=128)


@dataclasses.dataclass
class W4Tensor:
    """Canonical packed int4 tensor: ``packed[..., N, K/2]`` u8, ``scales[..., N, K/g]`` fp16 bits."""
    packed: np.ndarray
    scales: np.ndarray

    @property
    def n(self) -> int:
        return self.packed.shape[-2]

    @property
    def k(self) -> int:
        return self.packed.shape[-1] * 2


def _zero_mean_lut() -> np.ndarray:
    b = np.arange(256)
    lo, hi = b & 15, b >> 4
    lo = np.where(lo == 8, 0, lo)
    hi = np.where(hi == 8, 0, hi)
    return (lo | (hi << 4)).astype(np.uint8)


ZERO_MEAN_LUT = _zero_mean_lut()


def w4_tensor(seed: int, tag: int, stag: int, lead: tuple, n: int, k: int, g: int,
              ids: tuple = (), scale_lo: float = 0.005, scale_hi: float = 0.02, codes: str = "uniform") -> W4Tensor:
    """int4 codes and fp16 scales ~ U(lo, hi) (float64 draw, RNE).

    codes="uniform": every code in [-8, 7] equally likely (mean -1/2).
    codes="zero_mean": the uniform draw with code -8 replaced by 0, so codes
    lie in [-7, 7], symmetric, mean 0 (P(0) = 2/16, the others 1/16 each)."""
    shape = tuple(lead) + (n, k // 2)
    nbytes = int(np.prod(shape))
    lut = ZERO_MEAN_LUT if codes == "zero_mean" else None
    assert codes in ("uniform", "zero_mean")
    packed = splitmix_bytes(splitmix_key(seed, tag, *ids), nbytes, lut=lut).reshape(shape)
    scales = uniform_f16(rng(seed, stag, *ids), scale_lo, scale_hi, tuple(lead) + (n, k // g))
    return W4Tensor(packed, scales)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack int4 codes [..., K] (values in [-8, 7]) into the canonical byte layout [..., K/2]."""
    c = np.asarray(codes).astype(np.int64)
    assert c.shape[-1] % 2 == 0 and c.min() >= -8 and c.max() <= 7
    u = (c & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_codes` (storage format only)."""
    p = np.asarray(packed).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out


@dataclasses.dataclass
class LayerWeights:
    attn_norm: np.ndarray      # [H] fp16 bits
    qkv: W4Tensor              # [n_qkv, H]
    o: W4Tensor                # [H, q_dim]
    moe_norm: np.ndarray       # [H]
    router: W4Tensor           # [E, H]
    gate: W4Tensor             # [E, I, H]
    up: W4Tensor               # [E, I, H]
    down: W4Tensor             # [E, H, I]


@dataclasses.dataclass
class ModelWeights:
    desc: ModelDesc
    layers: list
    embed: W4Tensor | None     # [V, H]
    final_norm: np.ndarray | None
    lm_head: W4Tensor | None   # [V, H]


ONE_F16 = 0x3C00


def make_layer(desc: ModelDesc, seed: int, layer: int, codes: str = "uniform") -> LayerWeights:
    d, g = desc, desc.group
    H, E, I = d.hidden, d.n_experts, d.moe_inter
    ones = np.full(H, ONE_F16, dtype=np.uint16)    # RMSNorm gain 1 (random-init reading)
    c = dict(codes=codes)
    return LayerWeights(
        attn_norm=ones.copy(),
        qkv=w4_tensor(seed, T_QKV, T_QKV_S, (), d.n_qkv, H, g, (layer,), **c),
        o=w4_tensor(seed, T_O, T_O_S, (), H, d.q_dim, g, (layer,), **c),
        moe_norm=ones.copy(),
        router=w4_tensor(seed, T_ROUTER, T_ROUTER_S, (), E, H, g, (layer,), **c),
        gate=w4_tensor(seed, T_GATE, T_GATE_S, (E,), I, H, g, (layer,), **c),
        up=w4_tensor(seed, T_UP, T_UP_S, (E,), I, H, g, (layer,), **c),
        down=w4_tensor(seed, T_DOWN, T_DOWN_S, (E,), H, I, g, (layer,), **c),
    )


def make_model(desc: ModelDesc, seed: int = 0, with_vocab: bool = True, codes: str = "uniform") -> ModelWeights:
    """codes="zero_mean" is the full random-init model's reading: the uniform
    [-8, 7] draw has mean -1/2, which adds the same direction to every
    projection's output for every stream; through the layers it comes to
    dominate the router input and every stream picks the same few experts."""
    layers = [make_layer(desc, seed, l, codes) for l in range(desc.n_layers)]
    emb = lm = fn = None
    if with_vocab:
        emb = w4_tensor(seed, T_EMBED, T_EMBED_S, (), desc.vocab, desc.hidden, desc.group, codes=codes)
        lm = w4_tensor(seed, T_LM, T_LM_S, (), desc.vocab, desc.hidden, desc.group, codes=codes)
        fn = np.full(desc.hidden, ONE_F16, dtype=np.uint16)
    return ModelWeights(desc, layers, emb, fn, lm)


# --------------------------------------------------------------------------
# per-configuration activations and schedules
# --------------------------------------------------------------------------
def tiny_layer_case(seed: int = 0):
    """Tiny single MoE layer, one decode step: B=4 streams in an 8-slot x 128 arena,
    ragged positions {3, 17, 40, 64}; prefix KV ~ N(0,1) fp16 (taken as post-rotary)."""
    d = TINY
    g = rng(seed, T_X)
    x = normal_f16(g, (4, d.hidden))
    positions = np.array([3, 17, 40, 64], dtype=np.int32)
    slots = rng(seed, T_PERM).permutation(8)[:4].astype(np.int32)
    kv = []
    for b, p in enumerate(positions):
        gk = rng(seed, T_KV, b)
        k = normal_f16(gk, (d.n_layers, int(p), d.n_kv_heads, d.head_dim))
        v = normal_f16(gk, (d.n_layers, int(p), d.n_kv_heads, d.head_dim))
        kv.append((k, v))
    return dict(desc=d, x=x, positions=positions, slots=slots, kv=kv,
                n_slots=8, cap=128)


def dense_case(seed: int, B: int, n: int, k: int, g: int = 128, copy: int = 0):
    """Dense W4A16 projection: x fp16 [B,K] ~ N(0,1); W [N,K] int4, group g, scales ~U(0.005,0.02)."""
    x = normal_f16(rng(seed, T_X, B, n, k), (B, k))
    w = w4_tensor(seed, T_QKV, T_QKV_S, (), n, k, g, (n, k, copy))
    return x, w


def moe_logits(seed: int, B: int, E: int, regime: str, top_k: int = 8):
    """Router logits f32 [B,E].  'disjoint': i.i.d. N(0,1).  'skewed': a shared set of 6
    experts (+10) and 2 private experts per stream (+8, distinct across streams)."""
    g = rng(seed, T_LOGITS, B)
    base = g.standard_normal((B, E))
    if regime == "disjoint":
        return base.astype(np.float32), None
    assert regime == "skewed" and top_k == 8
    perm = g.permutation(E)
    shared = np.sort(perm[:6])
    rest = perm[6:]
    assert 2 * B <= len(rest)
    private = rest[: 2 * B].reshape(B, 2)
    lg = base.copy()
    lg[:, shared] += 10.0
    for b in range(B):
        lg[b, private[b]] += 8.0
    return lg.astype(np.float32), (shared, private)


def moe_case(seed: int, B: int, regime: str, desc: ModelDesc = FULL):
    x = normal_f16(rng(seed, T_X, B, 3), (B, desc.hidden))
    logits, extra = moe_logits(seed, B, desc.n_experts, regime, desc.top_k)
    return x, logits, extra


@dataclasses.dataclass
class Event:
    step: int
    kind: str            # "join" or "finish"
    stream: int
    prompt_len: int = 0
    life: int = 0


def ragged_schedule(seed: int, n_steps: int, max_streams: int, p_arrival: float,
                    prompt_max: int, life_lo: int, life_hi: int, first_join: int = 1):
    """Continuous-batching schedule.  Step 0 admits ``first_join`` streams; at each
    later step a request arrives with probability ``p_arrival`` (FIFO queue) and is
    admitted while a slot is free.  Prompt ~ U{1..prompt_max}; a stream decodes
    ``life`` ~ U{life_lo..life_hi} tokens, one per step, then finishes.

    Returns a list per step of the active stream ids (in admission order), plus a
    dict stream -> (prompt_len, life, join_step)."""
    g = rng(seed, T_SCHED)
    queue, active, info = [], [], {}
    nxt = 0
    per_step = []
    for s in range(n_steps):
        arrivals = first_join if s == 0 else int(g.random() < p_arrival)
        for _ in range(arrivals):
            info[nxt] = [int(g.integers(1, prompt_max + 1)), int(g.integers(life_lo, life_hi + 1)), -1]
            queue.append(nxt)
            nxt += 1
        while queue and len(active) < max_streams:
            sid = queue.pop(0)
            info[sid][2] = s
            active.append(sid)
        per_step.append(list(active))
        # each active stream decodes one token this step; retire finished ones
        done = [sid for sid in active if s - info[sid][2] + 1 >= info[sid][1]]
        for sid in done:
            active.remove(sid)
    return per_step, {k: tuple(v) for k, v in info.items()}


def attn_step_inputs(seed: int, step: int, B: int, desc_q: int, desc_kv: int, d: int):
    """q [B,Hq,D], k_new/v_new [B,Hkv,D] fp16 ~ N(0,1) for one attention step."""
    g = rng(seed, T_Q, step)
    q = normal_f16(g, (B, desc_q, d))
    k = normal_f16(g, (B, desc_kv, d))
    v = normal_f16(g, (B, desc_kv, d))
    return q, k, v


def prefix_kv(seed: int, stream: int, n_layers: int, prompt_len: int, n_kv: int, d: int):
    """Seeded prompt KV for one stream, canonical [layer][pos][kv_head][d] fp16 ~ N(0,1),
    taken as already rotary-embedded."""
    g = rng(seed, T_KV, stream)
    k = normal_f16(g, (n_layers, prompt_len, n_kv, d))
    v = normal_f16(g, (n_layers, prompt_len, n_kv, d))
    return k, v


def first_token(seed: int, stream: int, vocab: int) -> int:
    return int(rng(seed, T_TOKENS, stream).integers(0, vocab))
