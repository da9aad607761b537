"""Comparison helpers shared by the tests (no method arithmetic)."""
import numpy as np


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
