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
