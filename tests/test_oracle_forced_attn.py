"""Pins of two oracle entry points used as checkers on the GPU:

* the forced-routing input of the MoE block, the decoder layer and the whole
  step (a routing decision replayed at a near-tie of the k-th and (k+1)-th
  router logits): forcing the oracle's own choice changes nothing, bit for
  bit, and forcing any other ranked selection matches the float64 brute force
  given the same selection;
* the attention-only step with its KV append (slot-indexed GQA decode): the
  new key and value land at (layer, slot, position p) and nowhere else, and
  attention covers exactly positions 0..p, checked over a reused slot whose
  stale contents would change the result if a single extra or missing key were
  read."""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import ref64
from int4_w4a16_group_amd import inputs
from tests.util import assert_normwise, f16v, route_ok, ulp16

TOL = 2e-3


def tiny(layers=1, vocab=64, top_k=2, seed=0):
    d = dataclasses.replace(inputs.TINY, n_layers=layers, vocab=vocab, top_k=top_k)
    return d, inputs.make_model(d, seed, with_vocab=vocab > 0)


def _arena(case, d):
    ar = oracle.Arena(d, case["n_slots"], case["cap"])
    for b, (k, v) in enumerate(case["kv"]):
        ar.seed(int(case["slots"][b]), k, v)
    return ar


def _bottom_k(logits, k):
    """The k experts with the lowest logits, ranked by id descending: a selection
    no top-k rule would produce."""
    ids = np.argsort(logits, kind="stable")[:k]
    return np.sort(ids)[::-1].astype(np.int32)


# ------------------------------------------------------------------ forced routing
def test_route_weights_vs_fp64():
    g = inputs.rng(11, 1)
    logits = g.standard_normal((5, 8)).astype(np.float32) * 3
    ids = np.stack([g.permutation(8)[:3] for _ in range(5)]).astype(np.int32)
    w = oracle.route_weights(logits, ids)
    for b in range(5):
        ref = ref64.forced_weights(logits[b], ids[b])
        assert np.allclose(w[b], ref, rtol=1e-6, atol=0)
        assert abs(float(w[b].sum()) - 1.0) < 1e-6
    # the top-k's own weights are the same function of its ids
    tids, tw = oracle.topk_softmax(logits, 3)
    assert np.array_equal(oracle.route_weights(logits, tids), tw)


def test_forced_own_choice_is_bitwise_identity():
    case = inputs.tiny_layer_case(0)
    d = case["desc"]
    om = oracle.Model(inputs.make_model(d, 0, with_vocab=False))
    h0, ids0, lg0 = oracle.layer_step(om, _arena(case, d), 0, case["slots"], case["positions"], case["x"])
    h1, ids1, lg1 = oracle.layer_step(om, _arena(case, d), 0, case["slots"], case["positions"], case["x"],
                                      force=ids0)
    assert np.array_equal(h0, h1) and np.array_equal(ids0, ids1) and np.array_equal(lg0, lg1)
    # MoE block
    x, logits, _ = inputs.moe_case(0, 3, "disjoint", desc=d)
    y0, i0, w0 = oracle.moe(om, 0, x, logits)
    y1, i1, w1 = oracle.moe(om, 0, x, logits, force=i0)
    assert np.array_equal(y0, y1) and np.array_equal(w0, w1)
    # whole step, every layer forced to its own choice
    d2, mw2 = tiny(layers=2, vocab=64, seed=4)
    om2 = oracle.Model(mw2)
    a = oracle.Arena(d2, 2, 16)
    l0, n0, r0, _ = oracle.decode_step(om2, a, [0, 1], [0, 0], [3, 9])
    a = oracle.Arena(d2, 2, 16)
    l1, n1, r1, _ = oracle.decode_step(om2, a, [0, 1], [0, 0], [3, 9], force=r0)
    assert np.array_equal(l0, l1) and np.array_equal(n0, n1) and np.array_equal(r0, r1)


def test_forced_layer_vs_fp64():
    """A selection far from the top-k (the k lowest logits, reversed id order)
    is used as given, weighted by the softmax over its own logits."""
    case = inputs.tiny_layer_case(0)
    d = case["desc"]
    mw = inputs.make_model(d, 0, with_vocab=False)
    om = oracle.Model(mw)
    _, own, lg = oracle.layer_step(om, _arena(case, d), 0, case["slots"], case["positions"], case["x"])
    force = np.stack([_bottom_k(lg[b], d.top_k) for b in range(4)])
    assert all(set(force[b]).isdisjoint(own[b]) for b in range(4))
    h, ids, lg2 = oracle.layer_step(om, _arena(case, d), 0, case["slots"], case["positions"], case["x"],
                                    force=force)
    assert np.array_equal(ids, force) and np.array_equal(lg2, lg)
    for b in range(4):
        p = int(case["positions"][b])
        kc = np.zeros((case["cap"], d.n_kv_heads, d.head_dim))
        vc = np.zeros_like(kc)
        kc[:p] = f16v(case["kv"][b][0][0])
        vc[:p] = f16v(case["kv"][b][1][0])
        rh, rid, _ = ref64.layer(d, mw.layers[0], kc, vc, p, f16v(case["x"][b]), force_ids=force[b])
        assert list(rid) == list(force[b])
        assert_normwise(f16v(h[b]), rh, TOL, f"forced layer stream {b}")
        # and the unforced result is far from it: the forced ids are really used
        hu, _, _ = ref64.layer(d, mw.layers[0], kc.copy(), vc.copy(), p, f16v(case["x"][b]))
        assert np.max(np.abs(f16v(h[b]) - hu)) > 10 * TOL * np.max(np.abs(hu))


def test_forced_moe_and_decode_vs_fp64():
    d, mw = tiny(layers=2, vocab=64, seed=5)
    om = oracle.Model(mw)
    x, logits, _ = inputs.moe_case(2, 2, "disjoint", desc=d)
    force = np.stack([_bottom_k(logits[b], d.top_k) for b in range(2)])
    y, ids, w = oracle.moe(om, 1, x, logits, force=force)
    for b in range(2):
        r = ref64.moe(f16v(x[b]), force[b], ref64.forced_weights(logits[b], force[b]), mw.layers[1], d.group)
        assert_normwise(f16v(y[b]), r, TOL, f"forced moe row {b}")
    # whole step with layer 1 forced for stream 0 (layer 0 keeps its own choice)
    a = oracle.Arena(d, 1, 16)
    _, _, own, rl = oracle.decode_step(om, a, [0], [0], [17], want_router=True)
    f = own.copy()
    f[1, 0] = _bottom_k(rl[1, 0], d.top_k)
    a = oracle.Arena(d, 1, 16)
    lg, nx, ids, _ = oracle.decode_step(om, a, [0], [0], [17], force=f)
    assert np.array_equal(ids, f)
    kcs = [np.zeros((16, d.n_kv_heads, d.head_dim)) for _ in range(2)]
    vcs = [np.zeros((16, d.n_kv_heads, d.head_dim)) for _ in range(2)]
    rlog, _ = ref64.decode(d, mw, kcs, vcs, 0, 17, force_ids=f[:, 0])
    assert_normwise(f16v(lg[0]), rlog, TOL, "forced decode step")


def test_route_ok_accepts_near_ties_only():
    lg = np.array([5.0, 4.0, 3.0, 2.999, 1.0, -1.0], np.float32)
    assert route_ok([0, 1, 2], lg, TOL)                 # the exact top-3
    assert route_ok([0, 1, 3], lg, TOL)                 # 3.0 vs 2.999 is within 2e-3 * 5
    assert not route_ok([0, 1, 4], lg, TOL)             # 1.0 is not
    assert not route_ok([1, 0, 2], lg, TOL)             # rank order violated by a clear gap
    assert not route_ok([0, 0, 2], lg, TOL)             # duplicate expert


# ------------------------------------------------------------------ attention step with append
ATT = dataclasses.replace(inputs.TINY, n_layers=2)     # 4 q / 2 kv heads x 64


@pytest.mark.parametrize("positions", [(0, 63, 64), (64, 0, 127), (5, 100, 63)])
def test_attn_step_append_and_span_vs_fp64(positions):
    d = ATT
    Hq, Hkv, D = d.n_q_heads, d.n_kv_heads, d.head_dim
    n_slots, cap, layer = 4, 160, 1
    om = oracle.Model(inputs.make_model(d, 0, with_vocab=False))
    ar = oracle.Arena(d, n_slots, cap)
    g = inputs.rng(21, sum(positions))
    # a reused arena: every slot holds stale data of a previous stream (large
    # values, so one extra or missing key changes the output well beyond 1 ulp)
    ar.k[...] = inputs.f16_bits(4.0 * g.standard_normal(ar.k.shape))
    ar.v[...] = inputs.f16_bits(4.0 * g.standard_normal(ar.v.shape))
    slots = [2, 0, 3]
    B = len(slots)
    prefix = []
    for b, (s, p) in enumerate(zip(slots, positions)):
        k, v = inputs.prefix_kv(21, b, d.n_layers, p, Hkv, D)
        if p:
            ar.seed(s, k, v)
        prefix.append((k, v))
    before_k, before_v = ar.k.copy(), ar.v.copy()
    q = inputs.normal_f16(g, (B, Hq, D))
    kn = inputs.normal_f16(g, (B, Hkv, D))
    vn = inputs.normal_f16(g, (B, Hkv, D))
    o = oracle.attn_step(om, ar, layer, slots, list(positions), q, kn, vn)
    for b, (s, p) in enumerate(zip(slots, positions)):
        K = np.concatenate([f16v(prefix[b][0][layer]).reshape(p, Hkv, D), f16v(kn[b])[None]], 0)
        V = np.concatenate([f16v(prefix[b][1][layer]).reshape(p, Hkv, D), f16v(vn[b])[None]], 0)
        ref = ref64.attention(f16v(q[b]), K, V)
        got = f16v(o[b])
        # fp32 against fp64, each rounded once to fp16: equal or one fp16 unit apart
        assert np.all(np.abs(got - ref) <= ulp16(np.maximum(np.abs(got), np.abs(ref)))), (b, p)
        # the append: exactly (layer, slot, p) changed, to k_new / v_new
        assert np.array_equal(ar.k[layer, s, p], kn[b]) and np.array_equal(ar.v[layer, s, p], vn[b])
    changed = np.argwhere(np.any(ar.k != before_k, axis=(-1, -2)) | np.any(ar.v != before_v, axis=(-1, -2)))
    assert sorted(map(tuple, changed)) == sorted((layer, s, p) for s, p in zip(slots, positions))


def test_attn_step_catches_planted_span_errors():
    """The comparison above distinguishes p + 1 keys from p and from p + 2 keys,
    and an append at p from one at p + 1, on this data (so the pin has teeth)."""
    d = ATT
    Hq, Hkv, D = d.n_q_heads, d.n_kv_heads, d.head_dim
    g = inputs.rng(22, 0)
    p = 63
    K = f16v(inputs.f16_bits(4.0 * g.standard_normal((p + 2, Hkv, D))))
    V = f16v(inputs.f16_bits(4.0 * g.standard_normal((p + 2, Hkv, D))))
    q = f16v(inputs.normal_f16(g, (Hq, D)))
    good = ref64.attention(q, K[:p + 1], V[:p + 1])
    for bad in (ref64.attention(q, K[:p], V[:p]), ref64.attention(q, K[:p + 2], V[:p + 2]),
                ref64.attention(q, np.concatenate([K[:p], K[p + 1:p + 2]]), V[:p + 1])):
        assert np.any(np.abs(bad - good) > ulp16(np.maximum(np.abs(bad), np.abs(good))))
