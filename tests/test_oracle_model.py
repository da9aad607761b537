"""Pins of the oracle's MoE block, decoder layer and whole decode step: float64
brute force on tiny shapes, reductions to a single expert, and the batching
invariants (a stream's result does not depend on the batch, its slot, stale
arena contents, row order, or the run)."""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import ref64
from int4_w4a16_group_amd import inputs
from tests.util import assert_normwise, f16v

TOL = 2e-3


def tiny_model(layers=1, vocab=64, top_k=2, seed=0, **kw):
    d = dataclasses.replace(inputs.TINY, n_layers=layers, vocab=vocab, top_k=top_k, **kw)
    return d, inputs.make_model(d, seed)


def routing_gap_ok(logits, ids_a, ids_b, k, tol=TOL):
    """Equal top-k sets, or a near-tie at the k-th/(k+1)-th logit."""
    if set(ids_a) == set(ids_b):
        return True
    s = np.sort(logits)[::-1]
    return s[k - 1] - s[k] <= tol * np.abs(logits).max()


# ------------------------------------------------------------------ MoE
def test_moe_identical_experts_reduce_to_one_expert():
    d, mw = tiny_model()
    lw = mw.layers[0]
    for t in (lw.gate, lw.up, lw.down):
        t.packed[:] = t.packed[0:1]
        t.scales[:] = t.scales[0:1]
    om = oracle.Model(mw)
    x = inputs.normal_f16(inputs.rng(1, 2), (3, d.hidden))
    logits = inputs.rng(1, 3).standard_normal((3, d.n_experts)).astype(np.float32)
    y, ids, w = oracle.moe(om, 0, x, logits)
    one = np.stack([oracle.moe(om, 0, x[b:b + 1], np.eye(d.n_experts, dtype=np.float32)[[0]] * 50)[0][0]
                    for b in range(3)])
    assert np.array_equal(y, one)
    for b in range(3):
        r = ref64.expert_mlp(f16v(x[b]), ref64._Sub(lw.gate.packed[0], lw.gate.scales[0]),
                             ref64._Sub(lw.up.packed[0], lw.up.scales[0]),
                             ref64._Sub(lw.down.packed[0], lw.down.scales[0]), d.group)
        assert_normwise(f16v(y[b]), r, TOL, "identical experts vs fp64 expert")


def test_moe_top1_is_single_expert_mlp():
    d, mw = tiny_model(top_k=1)
    om = oracle.Model(mw)
    x = inputs.normal_f16(inputs.rng(2, 2), (4, d.hidden))
    logits = inputs.rng(2, 3).standard_normal((4, d.n_experts)).astype(np.float32)
    y, ids, w = oracle.moe(om, 0, x, logits)
    lw = mw.layers[0]
    for b in range(4):
        e = int(np.argmax(logits[b]))
        assert ids[b, 0] == e and w[b, 0] == 1.0
        r = ref64.expert_mlp(f16v(x[b]), ref64._Sub(lw.gate.packed[e], lw.gate.scales[e]),
                             ref64._Sub(lw.up.packed[e], lw.up.scales[e]),
                             ref64._Sub(lw.down.packed[e], lw.down.scales[e]), d.group)
        assert_normwise(f16v(y[b]), r, TOL, "top-1 vs fp64 expert")


@pytest.mark.parametrize("regime", ["disjoint", "skewed"])
def test_moe_full_shape_vs_fp64(regime):
    """Grouped-expert layer at its real sizes (hidden 2048, 128 experts, top-8,
    intermediate 768, group 128), two streams, against the float64 brute force."""
    d = inputs.FULL
    lw = inputs.make_layer(d, 0, 0)
    mw = inputs.ModelWeights(dataclasses.replace(d, n_layers=1), [lw], None, None, None)
    om = oracle.Model(mw)
    x, logits, extra = inputs.moe_case(0, 2, regime)
    y, ids, w = oracle.moe(om, 0, x, logits)
    for b in range(2):
        rid, rw = ref64.topk_softmax(logits[b], d.top_k)
        assert list(rid) == list(ids[b])
        if regime == "skewed":
            shared, private = extra
            assert set(ids[b]) == set(shared) | set(private[b])
        r = ref64.moe(f16v(x[b]), rid, rw, lw, d.group)
        assert_normwise(f16v(y[b]), r, TOL, "moe vs fp64")


# ------------------------------------------------------------------ layer
def _tiny_arena(case, d, fill=0.0):
    ar = oracle.Arena(d, case["n_slots"], case["cap"], fill=fill)
    for b, (k, v) in enumerate(case["kv"]):
        ar.seed(int(case["slots"][b]), k, v)
    return ar


def test_layer_tiny_vs_fp64():
    case = inputs.tiny_layer_case(0)
    d = case["desc"]
    mw = inputs.make_model(d, 0, with_vocab=False)
    om = oracle.Model(mw)
    ar = _tiny_arena(case, d)
    h, ids, lg = oracle.layer_step(om, ar, 0, case["slots"], case["positions"], case["x"])
    for b in range(4):
        p = int(case["positions"][b])
        kc = np.zeros((case["cap"], d.n_kv_heads, d.head_dim))
        vc = np.zeros_like(kc)
        kc[:p] = f16v(case["kv"][b][0][0])
        vc[:p] = f16v(case["kv"][b][1][0])
        rh, rid, rlg = ref64.layer(d, mw.layers[0], kc, vc, p, f16v(case["x"][b]))
        assert routing_gap_ok(lg[b], ids[b], rid, d.top_k)
        if set(ids[b]) == set(rid):
            assert_normwise(f16v(h[b]), rh, TOL, f"layer stream {b}")
        # new K/V written at the stream's own slot and position
        s = int(case["slots"][b])
        assert_normwise(f16v(ar.k[0, s, p]).ravel(), kc[p].ravel(), TOL, "appended K")
        assert_normwise(f16v(ar.v[0, s, p]).ravel(), vc[p].ravel(), TOL, "appended V")


def test_layer_batch_invariants_bitwise():
    """I1 batch vs alone, I2 slot id, I3 stale slot contents (NaN-poisoned),
    I5 row permutation, I6 repeat: all bit-identical in the oracle."""
    case = inputs.tiny_layer_case(0)
    d = case["desc"]
    om = oracle.Model(inputs.make_model(d, 0, with_vocab=False))
    x, pos, slots = case["x"], case["positions"], case["slots"]
    h_batch, _, _ = oracle.layer_step(om, _tiny_arena(case, d), 0, slots, pos, x)
    for b in range(4):                                           # I1
        ar = _tiny_arena(case, d)
        hb, _, _ = oracle.layer_step(om, ar, 0, slots[b:b + 1], pos[b:b + 1], x[b:b + 1])
        assert np.array_equal(hb[0], h_batch[b])
    moved = (slots + 3) % 8                                       # I2
    case2 = dict(case, slots=moved)
    h2, _, _ = oracle.layer_step(om, _tiny_arena(case2, d), 0, moved, pos, x)
    assert np.array_equal(h2, h_batch)
    ar3 = _tiny_arena(case, d, fill=np.nan)                      # I3: stale region is NaN
    h3, _, _ = oracle.layer_step(om, ar3, 0, slots, pos, x)
    assert np.array_equal(h3, h_batch)
    perm = np.array([2, 0, 3, 1])                                 # I5
    h5, _, _ = oracle.layer_step(om, _tiny_arena(case, d), 0, slots[perm], pos[perm], x[perm])
    assert np.array_equal(h5, h_batch[perm])
    h6, _, _ = oracle.layer_step(om, _tiny_arena(case, d), 0, slots, pos, x)   # I6
    assert np.array_equal(h6, h_batch)


# ------------------------------------------------------------------ whole step
def test_decode_step_tiny_model_vs_fp64():
    d, mw = tiny_model(layers=2, vocab=64, top_k=2, seed=3)
    om = oracle.Model(mw)
    cap = 32
    positions = np.array([0, 5, 11], np.int32)
    slots = np.array([2, 0, 1], np.int32)
    tokens = np.array([7, 63, 0], np.int32)
    ar = oracle.Arena(d, 3, cap)
    pre = []
    for b, p in enumerate(positions):
        k, v = inputs.prefix_kv(3, b, d.n_layers, int(p), d.n_kv_heads, d.head_dim)
        ar.seed(int(slots[b]), k, v)
        pre.append((k, v))
    logits, nxt, ids, _ = oracle.decode_step(om, ar, slots, positions, tokens)
    for b, p in enumerate(positions):
        kcs = [np.zeros((cap, d.n_kv_heads, d.head_dim)) for _ in range(d.n_layers)]
        vcs = [np.zeros((cap, d.n_kv_heads, d.head_dim)) for _ in range(d.n_layers)]
        for l in range(d.n_layers):
            kcs[l][:p] = f16v(pre[b][0][l])
            vcs[l][:p] = f16v(pre[b][1][l])
        rl, rt = ref64.decode(d, mw, kcs, vcs, int(p), int(tokens[b]))
        assert_normwise(f16v(logits[b]), rl, TOL, f"logits stream {b}")
        srt = np.sort(rl)[::-1]
        if srt[0] - srt[1] > TOL * np.abs(rl).max():
            assert nxt[b] == rt
        assert nxt[b] == int(np.argmax(f16v(logits[b])))


def test_decode_step_argmax_takes_lowest_id_on_ties():
    """All output-projection codes zero: every logit is 0 and the token is id 0."""
    d, mw = tiny_model(layers=1, vocab=32)
    mw.lm_head.packed[:] = 0
    om = oracle.Model(mw)
    ar = oracle.Arena(d, 1, 16)
    logits, nxt, _, _ = oracle.decode_step(om, ar, [0], [0], [5])
    assert np.all(f16v(logits) == 0) and nxt[0] == 0
