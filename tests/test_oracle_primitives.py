"""Pins of the CPU oracle's primitives against things other than itself:
IEEE binary16 as NumPy implements it, hand-worked fixtures, closed forms,
textbook special cases, float64 brute force and exhaustive small cases."""
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle import ref64
from int4_w4a16_group_amd import inputs
from tests.util import f16v, ulp16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture(name):
    d = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split(":", 1)
            d[k.strip()] = v.split()
    return d


def bits(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


# ------------------------------------------------------------------ fp16
def test_h2f_exhaustive_matches_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.h2f(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f2h_round_to_nearest_even():
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)     # all finite non-negative halves
    v = h.view(np.float16).astype(np.float64)
    nxt = np.append(v[1:], 65536.0)
    mid = (v + nxt) / 2                                               # exact ties (fit in float32)
    cases = [v, mid, np.nextafter(mid.astype(np.float32), np.float32(np.inf)).astype(np.float64),
             np.nextafter(mid.astype(np.float32), np.float32(0)).astype(np.float64)]
    g = np.random.default_rng(7)
    cases.append(np.exp(g.uniform(np.log(1e-9), np.log(7e4), 200000)))
    cases.append(np.array([65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -26]))
    for c in cases:
        c32 = np.concatenate([c, -c]).astype(np.float32)
        got = oracle.f2h(c32)
        ref = c32.astype(np.float16).view(np.uint16)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, f"{c32[bad[:5]]}: {got[bad[:5]]} vs {ref[bad[:5]]}"


# ------------------------------------------------------------------ int4 W4A16
def test_gemm_handworked_fixture():
    fx = _fixture("w4_gemm_handworked.txt")
    K, g = int(fx["K"][0]), int(fx["group"][0])
    packed = np.array([int(t, 16) for t in fx["packed"]], np.uint8).reshape(2, K // 2)
    scales = bits([float(t) for t in fx["scales"]]).reshape(2, K // g)
    x = bits([float(t) for t in fx["x"]]).reshape(1, K)
    y = oracle.w4_gemm(x, packed, scales, g)
    assert np.array_equal(f16v(y)[0], np.array([float(t) for t in fx["y"]]))


def test_gemm_one_hot_recovers_every_code_and_scale():
    """x = e_k gives y_n = fp16(q[n][k] * s[n][k/g]) exactly: pins nibble order,
    two's complement and scale indexing for all 16 codes at several scales."""
    g = 8
    N, K = 16, 32
    codes = np.array([[((n + k) % 16) - 8 for k in range(K)] for n in range(N)])
    packed = inputs.pack_codes(codes)
    sv = np.array([[0.005 * (1 + n) * (1 + j) for j in range(K // g)] for n in range(N)])
    scales = bits(sv)
    svals = f16v(scales)
    X = np.eye(K)
    y = f16v(oracle.w4_gemm(bits(X), packed, scales, g))
    want = codes.T * np.repeat(svals, g, axis=1).T                  # [K, N]
    assert np.array_equal(y, want.astype(np.float16).astype(np.float64))


def test_gemm_explicit_bytes():
    """A byte 0xE1 holds code 1 (low nibble) then code -2 (high nibble)."""
    row = np.array([0xE1, 0x87], np.uint8)
    assert [oracle.code_at(row, k) for k in range(4)] == [1, -2, 7, -8]


@pytest.mark.parametrize("B,N,K,g", [(3, 48, 256, 32), (2, 32, 512, 128), (1, 16, 768, 128)])
def test_gemm_vs_float64_error_bound(B, N, K, g):
    """Before the fp16 store |y32 - y64| <= gamma_K * sum|x w| (sequential fp32
    summation bound); the stored fp16 is then the RNE of y32."""
    x, w = inputs.dense_case(11, B, N, K, g)
    y32 = oracle.w4_gemm(x, w.packed, w.scales, g, out="f32").astype(np.float64)
    y16 = f16v(oracle.w4_gemm(x, w.packed, w.scales, g))
    xf = f16v(x)
    W = ref64.dequant(w.packed, w.scales, g)
    y64 = ref64.gemm(xf, w.packed, w.scales, g)
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    bound = gamma * (np.abs(xf) @ np.abs(W).T)
    assert np.all(np.abs(y32 - y64) <= bound)
    assert np.array_equal(y16, y32.astype(np.float16).astype(np.float64))
    assert np.all(np.abs(y16 - y64) <= bound + ulp16(y64) / 2 * (1 + 1e-12))


def test_gemm_single_group_constant_scale_is_matmul():
    """g = K and one scale per row: the product is s_n * (x . q_n), a plain matmul."""
    B, N, K = 4, 32, 128
    rg = np.random.default_rng(3)
    codes = rg.integers(-8, 8, (N, K))
    x = bits(rg.standard_normal((B, K)))
    s = bits(np.full((N, 1), 0.015625))                              # 2^-6: exact everywhere
    y = f16v(oracle.w4_gemm(x, inputs.pack_codes(codes), s, K, out="f16"))
    ref = (f16v(x) @ codes.T.astype(np.float64)) * 0.015625
    assert np.array_equal(y, ref.astype(np.float16).astype(np.float64))


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_unit_rms_and_fp64():
    rg = np.random.default_rng(5)
    x = bits(rg.standard_normal((6, 2048)) * 3)
    gamma = bits(np.ones(2048))
    y = f16v(oracle.rmsnorm(x, gamma, 1e-6))
    rms = np.sqrt(np.mean(y * y, axis=1))
    assert np.all(np.abs(rms - 1) < 1e-3)
    r = ref64.rmsnorm(f16v(x), 1.0, 1e-6)
    assert np.all(np.abs(y - r) <= ulp16(r))


def test_rmsnorm_gain_applies_per_channel():
    rg = np.random.default_rng(6)
    x = bits(rg.standard_normal((2, 256)))
    gam = bits(rg.uniform(0.5, 2.0, 256))
    y = f16v(oracle.rmsnorm(x, gam, 1e-6))
    r = ref64.rmsnorm(f16v(x), f16v(gam), 1e-6)
    assert np.all(np.abs(y - r) <= ulp16(r))


# ------------------------------------------------------------------ rotary
def test_rope_position_zero_is_identity():
    x = bits(np.random.default_rng(1).standard_normal((4, 64)))
    assert np.array_equal(oracle.rope(x, 0, 1e4), x)


def test_rope_preserves_pair_norms_and_matches_fp64():
    rg = np.random.default_rng(2)
    x = bits(rg.standard_normal((8, 128)))
    for p in (1, 17, 4095):
        y = f16v(oracle.rope(x, p, 1e4))
        xv = f16v(x)
        n0 = xv[:, :64] ** 2 + xv[:, 64:] ** 2
        n1 = y[:, :64] ** 2 + y[:, 64:] ** 2
        assert np.allclose(n0, n1, rtol=3e-3, atol=1e-3)
        r = ref64.rope(xv, p, 1e4)
        assert np.all(np.abs(y - r) <= ulp16(r))


def test_rope_rotates_the_right_pairs():
    """Unit vector e_i at position p: lands on (cos, sin) of angle p*base^(-2i/D) in (i, i+D/2)."""
    D = 16
    for i in range(D // 2):
        x = np.zeros((1, D))
        x[0, i] = 1.0
        p = 3
        y = f16v(oracle.rope(bits(x), p, 1e4))[0]
        ang = p * 1e4 ** (-2 * i / D)
        want = np.zeros(D)
        want[i], want[i + D // 2] = np.cos(ang), np.sin(ang)
        assert np.all(np.abs(y - want) <= ulp16(want))


def test_rope_scores_depend_on_relative_position():
    rg = np.random.default_rng(4)
    q = bits(rg.standard_normal((1, 64)))
    k = bits(rg.standard_normal((1, 64)))
    dots = []
    for p, pk in ((5, 2), (105, 102), (1003, 1000)):
        qr, kr = f16v(oracle.rope(q, p, 1e4)), f16v(oracle.rope(k, pk, 1e4))
        dots.append(float(qr[0] @ kr[0]))
    assert max(dots) - min(dots) < 0.02 * np.abs(f16v(q)).sum()


# ------------------------------------------------------------------ attention
def test_attention_handworked_fixture():
    fx = _fixture("attention_handworked.txt")
    q = bits([float(t) for t in fx["q"]]).reshape(1, 4)
    k = bits([float(t) for t in fx["k"]]).reshape(2, 1, 4)
    v = bits([float(t) for t in fx["v"]]).reshape(2, 1, 4)
    o = f16v(oracle.attention(q, k, v))[0]
    want = np.array([float(t) for t in fx["o"]])
    assert np.all(np.abs(o - want) <= ulp16(want) / 2 + 1e-6)


def test_attention_single_position_returns_v0():
    rg = np.random.default_rng(8)
    q = bits(rg.standard_normal((8, 128)))
    k = bits(rg.standard_normal((1, 1, 128)))
    v = bits(rg.standard_normal((1, 1, 128)))
    o = oracle.attention(q, k, v)
    assert np.array_equal(o, np.repeat(v[0], 8, axis=0))


def test_attention_equal_keys_average_values_and_bounds():
    rg = np.random.default_rng(9)
    npos = 37
    q = bits(rg.standard_normal((4, 64)))
    k = np.repeat(bits(rg.standard_normal((1, 2, 64))), npos, axis=0)
    v = bits(rg.standard_normal((npos, 2, 64)))
    o = f16v(oracle.attention(q, k, v))
    vv = f16v(v)
    for h in range(4):
        g = h * 2 // 4
        mean = vv[:, g, :].mean(axis=0)
        assert np.all(np.abs(o[h] - mean) <= ulp16(mean) + 1e-6)
    k2 = bits(rg.standard_normal((npos, 2, 64)) * 3)
    o2 = f16v(oracle.attention(q, k2, v))
    for h in range(4):
        g = h * 2 // 4
        assert np.all(o2[h] <= vv[:, g, :].max(axis=0) + 1e-6)
        assert np.all(o2[h] >= vv[:, g, :].min(axis=0) - 1e-6)


def test_attention_mha_matches_textbook_fp64():
    rg = np.random.default_rng(10)
    H, D, npos = 4, 64, 50
    q = bits(rg.standard_normal((H, D)))
    k = bits(rg.standard_normal((npos, H, D)))
    v = bits(rg.standard_normal((npos, H, D)))
    o = f16v(oracle.attention(q, k, v))
    Q, K, V = f16v(q), f16v(k), f16v(v)
    for h in range(H):
        s = K[:, h, :] @ Q[h] / np.sqrt(D)
        p = np.exp(s - s.max())
        p /= p.sum()
        want = p @ V[:, h, :]
        assert np.all(np.abs(o[h] - want) <= ulp16(want) / 2 + 1e-5 * np.abs(V).max())


def test_attention_gqa_head_mapping():
    """q head h reads kv head floor(h*Hkv/Hq): V of kv head g is the constant g+1."""
    Hq, Hkv, D, npos = 8, 2, 16, 5
    rg = np.random.default_rng(12)
    q = bits(rg.standard_normal((Hq, D)))
    k = bits(rg.standard_normal((npos, Hkv, D)))
    v = np.zeros((npos, Hkv, D))
    for g in range(Hkv):
        v[:, g, :] = g + 1
    o = f16v(oracle.attention(q, k, bits(v)))
    for h in range(Hq):
        assert np.all(o[h] == (h * Hkv) // Hq + 1)


# ------------------------------------------------------------------ routing
def test_topk_full_softmax_when_k_equals_E():
    from scipy.special import softmax
    rg = np.random.default_rng(13)
    lg = rg.standard_normal((5, 16)).astype(np.float32)
    ids, w = oracle.topk_softmax(lg, 16)
    for b in range(5):
        ref = softmax(lg[b].astype(np.float64))
        assert np.allclose(w[b], ref[ids[b]], rtol=1e-6, atol=1e-7)
        assert np.all(np.diff(lg[b][ids[b]]) <= 0)


def test_topk_k1_is_argmax_with_weight_one():
    rg = np.random.default_rng(14)
    lg = rg.standard_normal((20, 128)).astype(np.float32)
    ids, w = oracle.topk_softmax(lg, 1)
    assert np.array_equal(ids[:, 0], np.argmax(lg, axis=1))
    assert np.all(w == 1.0)


def test_topk_weights_sum_to_one_and_ties_take_lower_id():
    rg = np.random.default_rng(15)
    lg = rg.standard_normal((50, 128)).astype(np.float32)
    _, w = oracle.topk_softmax(lg, 8)
    assert np.all(np.abs(w.sum(axis=1) - 1) < 1e-6)
    tie = np.zeros((1, 8), np.float32)
    tie[0, [1, 3, 6]] = 2.0
    ids, w = oracle.topk_softmax(tie, 4)
    assert list(ids[0]) == [1, 3, 6, 0]
    assert np.allclose(w[0, :3], w[0, 0])


def test_topk_brute_force_all_orderings():
    """E = 4: every ordering of distinct logits and every tie pattern from {0,1,2}."""
    base = np.array([0.5, -1.0, 2.0, 1.25], np.float32)
    cases = [np.array(p, np.float32) for p in itertools.permutations(base)]
    cases += [np.array(c, np.float32) for c in itertools.product([0.0, 1.0, 2.0], repeat=4)]
    for lg in cases:
        for k in range(1, 5):
            ids, w = oracle.topk_softmax(lg[None], k)
            want = sorted(range(4), key=lambda e: (-float(lg[e]), e))[:k]
            assert list(ids[0]) == want
            rid, rw = ref64.topk_softmax(lg, k)
            assert list(rid) == want
            assert np.allclose(w[0], rw, rtol=1e-6)


def test_bucket_is_stable_sort_by_expert():
    rg = np.random.default_rng(16)
    for B, k, E in ((1, 8, 128), (7, 8, 128), (32, 8, 128), (4, 2, 8)):
        ids = np.stack([rg.permutation(E)[:k] for _ in range(B)]).astype(np.int32)
        counts, offsets, ps, pr = oracle.bucket(ids, E)
        flat = ids.reshape(-1)
        order = np.argsort(flat, kind="stable")
        assert np.array_equal(ps, order // k) and np.array_equal(pr, order % k)
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
