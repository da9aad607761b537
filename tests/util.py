"""Comparison helpers shared by the tests (no method arithmetic)."""
import numpy as np

from oracle import route_ok  # noqa: F401  (near-tie acceptance of a routing decision)


def f16v(bits) -> np.ndarray:
    """fp16 bit patterns -> float64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def normwise_err(got, ref) -> np.ndarray:
    """Per row: max_i |got_i - ref_i| / max_i |ref_i| (the normwise-infinity relative error)."""
    got = np.atleast_2d(np.asarray(got, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return num / np.where(den == 0, 1.0, den)


def assert_normwise(got, ref, tol, what=""):
    e = normwise_err(got, ref)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{what}: non-finite output"
    assert e.max() <= tol, f"{what}: normwise error {e.max():.3e} > {tol:.1e} (rows {np.argsort(-e)[:4]})"
    return e


def ulp16(v) -> np.ndarray:
    """Spacing of fp16 values at |v| (subnormal spacing below 2^-14)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def gemm_abs_sum(x_bits, packed, scales, group) -> np.ndarray:
    """sum_k |x_k| |w_nk| per output (for summation-order error bounds)."""
    p = np.asarray(packed).astype(np.int16)
    q = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.float64)
    lo, hi = p & 15, (p >> 4) & 15
    q[..., 0::2] = np.where(lo > 7, lo - 16, lo)
    q[..., 1::2] = np.where(hi > 7, hi - 16, hi)
    s = np.repeat(f16v(scales), group, axis=-1)
    return np.abs(f16v(x_bits)) @ np.abs(q * s).T


def assert_within_reorder_bound(got_bits, ref_bits, abs_sum, K, what=""):
    """Two fp32 summations of the same K products, each rounded once to fp16:
    |got - ref| <= 2 gamma_K sum|x w| + one fp16 ulp (Higham's bound per side)."""
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    g, r = f16v(got_bits), f16v(ref_bits)
    lim = 2 * gamma * abs_sum + ulp16(np.maximum(np.abs(g), np.abs(r)))
    bad = np.abs(g - r) > lim
    assert not bad.any(), f"{what}: {bad.sum()} outputs beyond the summation bound"

