"""Pins of the oracle's non-greedy sampler (temperature, top-k, top-p with a
counter-based draw): the published SplitMix64 sequence of its generator,
the greedy special cases, agreement with an independent float64
restatement of the same five steps, and the sampled frequencies against the
closed-form nucleus distribution (a chi-square test over 40000 draws, which a
wrong temperature, a missing renormalisation or an off-by-one in the nucleus
cut fails)."""
import numpy as np
import pytest

import oracle
from int4_w4a16_group_amd import inputs


def test_generator_is_published_splitmix64():
    # reference outputs of splitmix64 seeded with 1234567 (Vigna's splitmix64.c)
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert [oracle.splitmix(1234567, p) for p in range(5)] == want
    u = [oracle.draw(1234567, p) for p in range(5)]
    assert u == [(w >> 40) / 2.0 ** 24 for w in want]
    assert all(0.0 <= x < 1.0 for x in u)


def f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def ref_sample(bits, T, k, p, u):
    """Float64 restatement: rank (value desc, id asc, NaN as -inf), keep k; greedy at T = 0
    or k = 1; weights exp((l_r - l_0)/T); nucleus prefix c_m >= p c_{k-1}; first r with
    u c_m < c_r.  Returns (id, distance of u c_m to the nearest boundary, relative)."""
    v = bits.view(np.float16).astype(np.float64)
    v = np.where(np.isnan(v), -np.inf, v)
    order = sorted(range(len(v)), key=lambda i: (-v[i], i))[:min(k, len(v))]
    if T == 0 or len(order) == 1:
        return order[0], np.inf
    e = np.exp((v[order] - v[order[0]]) / T)
    c = np.cumsum(e)
    m = int(np.argmax(c >= p * c[-1])) if np.any(c >= p * c[-1]) else len(c) - 1
    t = u * c[m]
    r = int(np.argmax(t < c[:m + 1])) if np.any(t < c[:m + 1]) else m
    return order[r], float(np.min(np.abs(c[:m + 1] - t)) / c[m])


def test_greedy_cases():
    g = inputs.rng(31, 0)
    row = f16(g.standard_normal(500) * 3)
    v = row.view(np.float16).astype(np.float64)
    am = int(np.argmax(v))
    for seed, pos in ((1, 0), (7, 99)):
        assert oracle.sample(row, 0.0, 64, 1.0, seed, pos) == am          # temperature 0
        assert oracle.sample(row, 1.7, 1, 1.0, seed, pos) == am           # top_k 1
        assert oracle.sample(row, 1.0, 64, 1e-9, seed, pos) == am         # nucleus of one rank
    tie = np.zeros(50, np.uint16)
    tie[[9, 4, 30]] = f16([2.0, 2.0, 2.0])
    assert oracle.sample(tie, 0.0, 8, 1.0, 3, 3) == 4                    # ties to the lower id
    nan = tie.copy()
    nan[1] = 0x7E00                                                     # NaN never wins
    assert oracle.sample(nan, 0.0, 8, 1.0, 3, 3) == 4


@pytest.mark.parametrize("T,k,p", [(1.0, 64, 1.0), (0.7, 20, 0.9), (1.8, 5, 0.5), (0.3, 64, 0.95)])
def test_sampler_vs_fp64_restatement(T, k, p):
    g = inputs.rng(32, k)
    mism = 0
    for trial in range(40):
        row = f16(g.standard_normal(1000) * 2.5)
        seed = int(g.integers(0, 2**63))
        for pos in (0, 1, 17, 4095):
            got = oracle.sample(row, T, k, p, seed, pos)
            want, gap = ref_sample(row, T, k, p, oracle.draw(seed, pos))
            if got != want:
                assert gap < 1e-5, (trial, pos, got, want, gap)      # only at a rounding boundary
                mism += 1
    assert mism <= 2


def test_sampled_frequencies_match_the_nucleus_distribution():
    logits = np.array([2.0, 1.5, 1.5, 0.25, -0.5, 3.0, -2.0, 0.75, 1.0, -1.0, 0.0, 2.5])
    row = f16(logits)
    T, k, p = 0.8, 6, 0.85
    v = row.view(np.float16).astype(np.float64)
    order = sorted(range(len(v)), key=lambda i: (-v[i], i))[:k]
    w = np.exp((v[order] - v[order[0]]) / T)
    cdf = np.cumsum(w) / w.sum()
    m = int(np.argmax(cdf >= p))
    prob = np.zeros(len(v))
    prob[order[:m + 1]] = w[:m + 1] / w[:m + 1].sum()
    n = 40000
    counts = np.bincount([oracle.sample(row, T, k, p, 20240601, pos) for pos in range(n)], minlength=len(v))
    assert np.all(counts[prob == 0] == 0)                              # nothing outside the nucleus
    exp = prob[prob > 0] * n
    chi2 = float(np.sum((counts[prob > 0] - exp) ** 2 / exp))
    dof = int(np.sum(prob > 0)) - 1
    from scipy.stats import chi2 as chi2_dist
    assert chi2_dist.sf(chi2, dof) > 1e-4, (chi2, dof, counts[prob > 0], exp)
    # the same test rejects a sampler that ignores the temperature
    wrong = np.exp(v[order] - v[order[0]])
    pw = np.zeros(len(v))
    pw[order[:m + 1]] = wrong[:m + 1] / wrong[:m + 1].sum()
    chi2w = float(np.sum((counts[pw > 0] - pw[pw > 0] * n) ** 2 / (pw[pw > 0] * n)))
    assert chi2_dist.sf(chi2w, dof) < 1e-6
