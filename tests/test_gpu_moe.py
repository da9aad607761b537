"""Grouped-expert MoE layer on the GPU against the oracle (hidden 2048, 128
experts, top-8, intermediate 768, group 128; B in {1, 4, 8, 32}; disjoint and
skewed routing).  Routing and bucketing are integer results and must match
exactly; expert outputs within the normwise tolerance; every stream's row
bit-identical to the same stream run alone."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from int4_w4a16_group_amd import _lib as L
from int4_w4a16_group_amd import inputs
from int4_w4a16_group_amd.engine import Context
from tests.gpu_util import empty_f16, to_dev, to_host
from tests.util import assert_normwise, f16v, route_ok

pytestmark = pytest.mark.gpu
TOL = 2e-3
MOE = dataclasses.replace(inputs.FULL, n_layers=1, vocab=16)


@pytest.fixture(scope="module")
def moe_ctx(gpu):
    lw = inputs.make_layer(MOE, 0, 0)
    ctx = Context(MOE, 32, 64)
    ctx.load_layer(0, lw)
    mw = inputs.ModelWeights(MOE, [lw], None, None, None)
    yield ctx, oracle.Model(mw)
    ctx.close()


def gpu_moe(ctx, x, logits, dev):
    B = x.shape[0]
    xd = to_dev(x, dev)
    ld = to_dev(logits, dev) if logits is not None else None
    y = empty_f16((B, MOE.hidden), dev)
    ids = torch.empty((B, MOE.top_k), dtype=torch.int32, device=dev)
    L.w4_moe(ctx.ctx, 0, B, xd, ld, y, ids, ctx.stream)
    return to_host(y), to_host(ids)


@pytest.mark.parametrize("regime", ["disjoint", "skewed"])
@pytest.mark.parametrize("B", [1, 4, 8, 32])
def test_moe_parity(moe_ctx, gpu, regime, B):
    ctx, om = moe_ctx
    x, logits, _ = inputs.moe_case(0, B, regime)
    y, ids = gpu_moe(ctx, x, logits, gpu)
    ry, rids, rw = oracle.moe(om, 0, x, logits)
    assert np.array_equal(ids, rids)
    assert_normwise(f16v(y), f16v(ry), TOL, f"moe B={B} {regime}")


@pytest.mark.parametrize("regime", ["disjoint", "skewed"])
def test_moe_rows_bit_identical_to_single_stream(moe_ctx, gpu, regime):
    ctx, _ = moe_ctx
    x, logits, _ = inputs.moe_case(1, 32, regime)
    y, _ = gpu_moe(ctx, x, logits, gpu)
    for b in (0, 5, 17, 31):
        y1, _ = gpu_moe(ctx, x[b:b + 1], logits[b:b + 1], gpu)
        assert np.array_equal(y1[0], y[b]), b
    perm = np.random.default_rng(3).permutation(32)
    yp, _ = gpu_moe(ctx, x[perm], logits[perm], gpu)
    assert np.array_equal(yp, y[perm])


@pytest.mark.parametrize("B", [1, 7, 32])
def test_route_and_bucketing_exact(moe_ctx, gpu, B):
    ctx, _ = moe_ctx
    E, k = MOE.n_experts, MOE.top_k
    logits, _ = inputs.moe_logits(2, B, E, "disjoint")
    logits[0, 5] = logits[0, 9] = logits[0].max() + 1.0          # an exact tie: lower id first
    ld = to_dev(logits, gpu)
    ids = torch.empty((B, k), dtype=torch.int32, device=gpu)
    w = torch.empty((B, k), dtype=torch.float32, device=gpu)
    counts = torch.empty(E, dtype=torch.int32, device=gpu)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=gpu)
    ps = torch.empty(B * k, dtype=torch.int32, device=gpu)
    pr = torch.empty(B * k, dtype=torch.int32, device=gpu)
    L.w4_route(ctx.ctx, B, ld, ids, w, counts, offsets, ps, pr, ctx.stream)
    rids, rw = oracle.topk_softmax(logits, k)
    assert np.array_equal(to_host(ids), rids)
    assert to_host(ids)[0, 0] == 5 and to_host(ids)[0, 1] == 9
    assert np.allclose(to_host(w), rw, rtol=2e-6, atol=1e-7)
    c, o, s, r = oracle.bucket(rids, E)
    assert np.array_equal(to_host(counts), c) and np.array_equal(to_host(offsets), o)
    assert np.array_equal(to_host(ps), s) and np.array_equal(to_host(pr), r)


def test_moe_router_computed_on_device(moe_ctx, gpu):
    """Logits from the layer's int4 router (fp32) instead of injected ones."""
    ctx, om = moe_ctx
    x = inputs.normal_f16(inputs.rng(4, 4), (6, MOE.hidden))
    y, ids = gpu_moe(ctx, x, None, gpu)
    mw_layer = inputs.make_layer(MOE, 0, 0)
    rl = oracle.w4_gemm(x, mw_layer.router.packed, mw_layer.router.scales, MOE.group, out="f32")
    # the oracle replays the GPU's routing once it is accepted as a top-k of the
    # oracle's logits (exactly the top-k unless the k-th and (k+1)-th are within
    # the tolerance), so every row is compared
    ry, rids, _ = oracle.moe(om, 0, x, rl, force=ids)
    for b in range(6):
        assert route_ok(ids[b], rl[b], TOL), f"row {b}: routing differs beyond a near-tie"
        assert_normwise(f16v(y[b]), f16v(ry[b]), TOL, f"router-on-device row {b}")


def moe_both_forms(ctx, x, logits, dev, layer=0):
    """w4_moe with the expert products as one launch and as two: (y, ids) each."""
    out = []
    for fused in (1, 0):
        L.w4_set_option(ctx.ctx, L.W4_OPT_FUSED_MOE, fused)
        B = x.shape[0]
        y = empty_f16((B, ctx.desc.hidden), dev)
        ids = torch.empty((B, ctx.desc.top_k), dtype=torch.int32, device=dev)
        L.w4_moe(ctx.ctx, layer, B, to_dev(x, dev), to_dev(logits, dev), y, ids, ctx.stream)
        out.append((to_host(y), to_host(ids)))
    L.w4_set_option(ctx.ctx, L.W4_OPT_FUSED_MOE, 0)
    L.w4_check_errors(ctx.ctx)   # no device-side wait ran out
    return out


@pytest.mark.parametrize("regime", ["disjoint", "skewed"])
@pytest.mark.parametrize("B", [1, 4, 8, 32])
def test_fused_expert_launch_matches_two_launches(moe_ctx, gpu, regime, B):
    """The one-launch expert products (gate/up, then down on per-unit
    completion counters) give the two-launch results bit for bit; run twice,
    so the counters are reused across calls."""
    ctx, _ = moe_ctx
    for seed in (5, 6):
        x, logits, _ = inputs.moe_case(seed, B, regime)
        (yf, idf), (y2, id2) = moe_both_forms(ctx, x, logits, gpu)
        assert np.array_equal(idf, id2)
        assert np.array_equal(yf, y2), f"B={B} {regime} seed {seed}"


@pytest.mark.parametrize("geom", [dict(), dict(moe_inter=128, n_experts=64, top_k=4),
                                  dict(moe_inter=256, group=64, n_experts=64, top_k=4), dict(hidden=1024)])
def test_fused_expert_launch_other_geometries(gpu, geom):
    """Other slice counts: gate/up over 8 or 4 waves, down over 1-3 waves in
    up to 8 sub-groups, other group sizes."""
    d = dataclasses.replace(inputs.FULL, n_layers=1, vocab=16, **geom)
    lw = inputs.make_layer(d, 3, 0)
    ctx = Context(d, 32, 64)
    try:
        ctx.load_layer(0, lw)
        for B in (1, 13, 32):
            x = inputs.normal_f16(inputs.rng(3, inputs.T_X, B, 9), (B, d.hidden))
            logits, _ = inputs.moe_logits(3, B, d.n_experts, "disjoint")
            (yf, idf), (y2, id2) = moe_both_forms(ctx, x, logits, gpu)
            assert np.array_equal(idf, id2) and np.array_equal(yf, y2), (geom, B)
    finally:
        ctx.close()


def test_fused_expert_launch_in_decode_steps(gpu):
    """Whole decode steps (3 layers, 6 streams, 3 steps) with the expert
    products as one launch and as two: the same logits bit for bit."""
    d = dataclasses.replace(inputs.FULL, n_layers=3, vocab=1000)
    mw = inputs.make_model(d, 8, codes="zero_mean")
    outs = []
    for fused in (1, 0):
        ctx = Context(d, 8, 256)
        try:
            ctx.load_model(mw)
            L.w4_set_option(ctx.ctx, L.W4_OPT_FUSED_MOE, fused)
            slots = []
            for s, p in enumerate((5, 64, 100, 1, 77, 130)):
                k, v = inputs.prefix_kv(8, s, d.n_layers, p, d.n_kv_heads, d.head_dim)
                slots.append(ctx.join(p, 8, k, v))
            tok = torch.tensor([3, 99, 500, 7, 42, 999], dtype=torch.int32, device=gpu)
            nxt = torch.empty(6, dtype=torch.int32, device=gpu)
            steps = []
            for _ in range(3):
                lg = empty_f16((6, d.vocab), gpu)
                L.w4_decode_step(ctx.ctx, slots, tok, lg, nxt, None, ctx.stream)
                steps.append(to_host(lg))
                tok, nxt = nxt.clone(), tok
            L.w4_check_errors(ctx.ctx)
            outs.append(steps)
        finally:
            ctx.close()
    for i, (a, b) in enumerate(zip(*outs)):
        assert np.array_equal(a, b), f"step {i}"


@pytest.mark.parametrize("P", [300, 1100])
def test_fused_expert_launch_in_prefill(gpu, P):
    """A 300- or 1100-token prompt (many 16-row units per expert) through a
    two-layer model with the expert products as one launch (16-row units) and
    as two (32-row units at 300 tokens, 64-row units at 1100): the same K/V,
    last logits and next id, bit for bit."""
    d = dataclasses.replace(inputs.FULL, n_layers=2, vocab=1000)
    mw = inputs.make_model(d, 9, codes="zero_mean")
    tokens = [int(t) for t in inputs.rng(9, inputs.T_TOKENS, 3).integers(0, d.vocab, P)]
    outs = []
    for fused in (1, 0):
        ctx = Context(d, 2, (P + 4 + 63) // 64 * 64)
        try:
            ctx.load_model(mw)
            L.w4_set_option(ctx.ctx, L.W4_OPT_FUSED_MOE, fused)
            lg = empty_f16((d.vocab,), gpu)
            nx = torch.empty(1, dtype=torch.int32, device=gpu)
            s = ctx.prefill(tokens, 4, lg, nx)
            k, v = ctx.read_kv(s)
            L.w4_check_errors(ctx.ctx)
            outs.append((k, v, to_host(lg), int(to_host(nx)[0])))
        finally:
            ctx.close()
    (k1, v1, l1, n1), (k2, v2, l2, n2) = outs
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2) and np.array_equal(l1, l2) and n1 == n2
