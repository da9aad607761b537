"""Float64 brute force of the int4 MoE decode step -- TEST INFRASTRUCTURE ONLY.

An independent NumPy restatement, used to pin the C oracle on small inputs.
Everything is float64 except the fp16 storage points, which are the same
as the oracle's (NumPy's float64 -> float16 cast rounds to nearest even).
It shares no code with the C oracle or with the GPU library.
"""
from __future__ import annotations

import numpy as np


def f16(a) -> np.ndarray:
    """Round float64 values to fp16 and return them as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def from_bits(h) -> np.ndarray:
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


def codes(packed: np.ndarray) -> np.ndarray:
    """int4 two's-complement codes; element 2j in the low nibble of byte j."""
    p = np.asarray(packed, dtype=np.int64)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return np.where(out > 7, out - 16, out)


def dequant(packed: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    q = codes(packed).astype(np.float64)
    s = from_bits(scales)
    return q * np.repeat(s, group, axis=-1)


def gemm(x: np.ndarray, packed, scales, group) -> np.ndarray:
    """x float64 [B,K]; returns the float64 product before any storage rounding."""
    W = dequant(packed, scales, group)
    B, K = x.shape
    y = np.zeros((B, W.shape[0]))
    for k in range(K):                      # explicit sum over k
        y += np.outer(x[:, k], W[:, k])
    return y


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return f16(x / np.sqrt(ms + eps) * gamma)


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """x float64 [nh, D]; rotate-half pairs (i, i + D/2)."""
    D = x.shape[-1]
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    ang = pos * theta ** (-2.0 * i / D)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return f16(np.concatenate([a * c - b * s, a * s + b * c], axis=-1))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q [Hq,D]; k, v [npos, Hkv, D] (float64) -> fp16-rounded [Hq, D]."""
    Hq, D = q.shape
    Hkv = k.shape[1]
    o = np.empty((Hq, D))
    for h in range(Hq):
        g = (h * Hkv) // Hq
        z = (k[:, g, :] @ q[h]) / np.sqrt(D)
        p = np.exp(z - z.max())
        p /= p.sum()
        o[h] = p @ v[:, g, :]
    return f16(o)


def topk_softmax(logits: np.ndarray, k: int):
    """Rank by (-logit, expert id); softmax over the k selected."""
    E = logits.shape[-1]
    order = sorted(range(E), key=lambda e: (-float(logits[e]), e))
    ids = np.array(order[:k])
    sel = logits[ids].astype(np.float64)
    w = np.exp(sel - sel.max())
    return ids, w / w.sum()


def forced_weights(logits: np.ndarray, ids) -> np.ndarray:
    """Softmax over the logits of a given ranked selection (a replayed routing decision)."""
    sel = np.asarray(logits, dtype=np.float64)[np.asarray(ids)]
    w = np.exp(sel - sel.max())
    return w / w.sum()


def expert_mlp(x: np.ndarray, gate, up, down, group) -> np.ndarray:
    """One SwiGLU expert on a float64 row x (already fp16-valued)."""
    g = f16(gemm(x[None], gate.packed, gate.scales, group)[0])
    u = f16(gemm(x[None], up.packed, up.scales, group)[0])
    a = f16(g / (1.0 + np.exp(-g)) * u)
    return f16(gemm(a[None], down.packed, down.scales, group)[0])


class _Sub:
    def __init__(self, packed, scales):
        self.packed, self.scales = packed, scales


def moe(x: np.ndarray, ids, w, lw, group) -> np.ndarray:
    """x float64 [H] (fp16-valued); experts of layer weights ``lw``."""
    acc = np.zeros_like(x)
    for r, e in enumerate(ids):
        y = expert_mlp(x, _Sub(lw.gate.packed[e], lw.gate.scales[e]),
                       _Sub(lw.up.packed[e], lw.up.scales[e]),
                       _Sub(lw.down.packed[e], lw.down.scales[e]), group)
        acc += w[r] * y
    return f16(acc)


def layer(desc, lw, kcache, vcache, pos: int, h: np.ndarray, force_ids=None):
    """One decoder layer for one stream.  kcache / vcache: float64 [cap, Hkv, D]
    holding positions 0..pos-1 (updated in place at pos).  h float64 [H].
    force_ids: ranked expert ids used instead of the router's top-k, or None."""
    d = desc
    nq, nkv = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    xn = rmsnorm(h, from_bits(lw.attn_norm), d.rms_eps)
    qkv = f16(gemm(xn[None], lw.qkv.packed, lw.qkv.scales, d.group)[0])
    q = rope(qkv[:nq].reshape(d.n_q_heads, d.head_dim), pos, d.rope_theta)
    k = rope(qkv[nq:nq + nkv].reshape(d.n_kv_heads, d.head_dim), pos, d.rope_theta)
    v = qkv[nq + nkv:].reshape(d.n_kv_heads, d.head_dim)
    kcache[pos], vcache[pos] = k, v
    att = attention(q, kcache[:pos + 1], vcache[:pos + 1]).reshape(-1)
    h = f16(h + f16(gemm(att[None], lw.o.packed, lw.o.scales, d.group)[0]))
    xn2 = rmsnorm(h, from_bits(lw.moe_norm), d.rms_eps)
    logits = gemm(xn2[None], lw.router.packed, lw.router.scales, d.group)[0]
    if force_ids is None:
        ids, w = topk_softmax(logits, d.top_k)
    else:
        ids = np.asarray(force_ids)
        w = forced_weights(logits, ids)
    h = f16(h + moe(xn2, ids, w, lw, d.group))
    return h, ids, logits


def decode(desc, mw, kcaches, vcaches, pos: int, token: int, force_ids=None):
    """Whole decode step for one stream; caches: per-layer float64 [cap, Hkv, D].
    force_ids: per layer ranked expert ids replacing the top-k, or None."""
    d = desc
    emb = dequant(mw.embed.packed[token], mw.embed.scales[token], d.group)
    h = f16(emb)
    for l, lw in enumerate(mw.layers):
        h, _, _ = layer(d, lw, kcaches[l], vcaches[l], pos, h, None if force_ids is None else force_ids[l])
    hn = rmsnorm(h, from_bits(mw.final_norm), d.rms_eps)
    logits = f16(gemm(hn[None], mw.lm_head.packed, mw.lm_head.scales, d.group)[0])
    return logits, int(np.argmax(logits))
