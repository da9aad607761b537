"""Pins of the oracle's prefill (a joining stream's prompt through the model,
causally, writing the slot's K/V): against the float64 brute force run token
by token over the prompt (K/V at every position and layer, and the last
token's logits), equal bit for bit to the same tokens fed as single decode
steps, and a no-op when its own routing is forced."""
import dataclasses

import numpy as np

import oracle
from oracle import ref64
from int4_w4a16_group_amd import inputs
from tests.util import assert_normwise, f16v

TOL = 2e-3


def tiny(layers=2, vocab=64, seed=6):
    d = dataclasses.replace(inputs.TINY, n_layers=layers, vocab=vocab, top_k=2)
    return d, inputs.make_model(d, seed)


def test_prefill_vs_fp64_token_by_token():
    d, mw = tiny()
    om = oracle.Model(mw)
    P, slot, cap = 6, 1, 16
    tokens = [5, 63, 0, 17, 17, 40]
    ar = oracle.Arena(d, 3, cap)
    logits, nxt, _ = oracle.prefill(om, ar, slot, tokens)
    kcs = [np.zeros((cap, d.n_kv_heads, d.head_dim)) for _ in range(d.n_layers)]
    vcs = [np.zeros((cap, d.n_kv_heads, d.head_dim)) for _ in range(d.n_layers)]
    for t in range(P):
        rl, rt = ref64.decode(d, mw, kcs, vcs, t, tokens[t])
    assert_normwise(f16v(logits), rl, TOL, "prefill logits")
    srt = np.sort(rl)[::-1]
    if srt[0] - srt[1] > TOL * np.abs(rl).max():
        assert nxt == rt
    for l in range(d.n_layers):
        for t in range(P):
            assert_normwise(f16v(ar.k[l, slot, t]).ravel(), kcs[l][t].ravel(), TOL, f"K layer {l} pos {t}")
            assert_normwise(f16v(ar.v[l, slot, t]).ravel(), vcs[l][t].ravel(), TOL, f"V layer {l} pos {t}")
    assert not np.any(ar.k[:, [0, 2]]) and not np.any(ar.k[:, slot, P:])      # nothing else written


def test_prefill_equals_single_decode_steps_and_forced_own_routing():
    d, mw = tiny(layers=3, vocab=80, seed=7)
    om = oracle.Model(mw)
    tokens = [int(t) for t in inputs.rng(7, 1).integers(0, d.vocab, 9)]
    a1 = oracle.Arena(d, 2, 16)
    l1, n1, ids1 = oracle.prefill(om, a1, 0, tokens, want_ids=True)
    a2 = oracle.Arena(d, 2, 16)
    for t, tok in enumerate(tokens):
        l2, n2, i2, _ = oracle.decode_step(om, a2, [0], [t], [tok])
        assert np.array_equal(i2[:, 0], ids1[:, t])
    assert np.array_equal(l1, l2[0]) and n1 == int(n2[0])
    assert np.array_equal(a1.k, a2.k) and np.array_equal(a1.v, a2.v)
    a3 = oracle.Arena(d, 2, 16)
    l3, n3, ids3 = oracle.prefill(om, a3, 0, tokens, force=ids1, want_ids=True)
    assert np.array_equal(l3, l1) and np.array_equal(a3.k, a1.k) and np.array_equal(ids3, ids1)
