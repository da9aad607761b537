"""Dense W4A16 projection on the GPU against the oracle: the fused q/k/v shape
(5120 x 2048) and the output projection (2048 x 4096) at B in {1..32}, group
128; plus ragged N (pad tiles), K that is not a multiple of 256, and groups
32/64.  Row results must be bit-identical across batch sizes and row orders."""
import dataclasses

import numpy as np
import pytest

import oracle
from int4_w4a16_group_amd import _lib as L
from int4_w4a16_group_amd import inputs
from int4_w4a16_group_amd.engine import Context
from tests.gpu_util import empty_f16, to_dev, to_host, ulp_diff
from tests.util import assert_normwise, assert_within_reorder_bound, f16v, gemm_abs_sum

pytestmark = pytest.mark.gpu
TOL = 2e-3
DENSE = dataclasses.replace(inputs.FULL, n_layers=1, n_experts=8, top_k=2, moe_inter=128, vocab=16)


@pytest.fixture(scope="module")
def dense_ctx(gpu):
    ctx = Context(DENSE, 32, 64)
    wq = inputs.w4_tensor(0, inputs.T_QKV, inputs.T_QKV_S, (), 5120, 2048, 128, (5120, 2048, 0))
    wo = inputs.w4_tensor(0, inputs.T_QKV, inputs.T_QKV_S, (), 2048, 4096, 128, (2048, 4096, 0))
    ctx.load_tensor(0, L.W4_T_QKV, 0, wq.packed, wq.scales)
    ctx.load_tensor(0, L.W4_T_O, 0, wo.packed, wo.scales)
    yield ctx, {L.W4_T_QKV: wq, L.W4_T_O: wo}
    ctx.close()


def run(ctx, tensor, x_bits, N, dev, expert=0, layer=0, f32=False):
    import torch
    B = x_bits.shape[0]
    x = to_dev(x_bits, dev)
    y = torch.empty((B, N), dtype=torch.float32, device=dev) if f32 else empty_f16((B, N), dev)
    L.w4_gemm(ctx.ctx, layer, tensor, expert, B, x, y, ctx.stream)
    return to_host(y)


@pytest.mark.parametrize("tensor,N,K", [(L.W4_T_QKV, 5120, 2048), (L.W4_T_O, 2048, 4096)])
def test_dense_projection_parity_and_batch_identity(dense_ctx, gpu, tensor, N, K):
    ctx, ws = dense_ctx
    w = ws[tensor]
    x32 = inputs.normal_f16(inputs.rng(0, inputs.T_X, N, K), (32, K))
    ref = oracle.w4_gemm(x32, w.packed, w.scales, 128)
    y32 = run(ctx, tensor, x32, N, gpu)
    assert_normwise(f16v(y32), f16v(ref), TOL, "dense vs oracle")
    assert_within_reorder_bound(y32, ref, gemm_abs_sum(x32, w.packed, w.scales, 128), K, "dense vs oracle")
    assert (ulp_diff(y32, ref) > 1).mean() < 1e-3
    for B in (1, 2, 4, 8, 16, 17):
        yb = run(ctx, tensor, x32[:B], N, gpu)
        assert np.array_equal(yb, y32[:B]), f"rows differ between B={B} and B=32"
    perm = np.random.default_rng(1).permutation(32)
    yp = run(ctx, tensor, x32[perm], N, gpu)
    assert np.array_equal(yp, y32[perm])


@pytest.mark.parametrize("N,K,g,B", [(200, 384, 32, 3), (136, 256, 64, 20), (48, 640, 128, 1), (512, 1024, 32, 32)])
def test_ragged_shapes_and_groups(gpu, N, K, g, B):
    """Output projection of a small model: N = vocab (pad rows), K = hidden."""
    d = dataclasses.replace(inputs.TINY, hidden=K, vocab=N, group=g)
    ctx = Context(d, 32, 64)
    try:
        w = inputs.w4_tensor(5, inputs.T_LM, inputs.T_LM_S, (), N, K, g)
        ctx.load_tensor(0, L.W4_T_LM_HEAD, 0, w.packed, w.scales)
        x = inputs.normal_f16(inputs.rng(5, N, K), (B, K))
        y = run(ctx, L.W4_T_LM_HEAD, x, N, gpu)
        ref = oracle.w4_gemm(x, w.packed, w.scales, g)
        assert_normwise(f16v(y), f16v(ref), TOL, "ragged vs oracle")
        assert_within_reorder_bound(y, ref, gemm_abs_sum(x, w.packed, w.scales, g), K, "ragged vs oracle")
        y1 = run(ctx, L.W4_T_LM_HEAD, x[-1:], N, gpu)
        assert np.array_equal(y1[0], y[-1])
    finally:
        ctx.close()


def test_one_hot_rows_recover_codes_times_scales(gpu):
    """x = e_k picks column k: y[n] = fp16(q[n][k] * s[n][k/g]) exactly (layout pin on the device)."""
    N, K, g = 64, 256, 32
    d = dataclasses.replace(inputs.TINY, hidden=K, vocab=N, group=g)
    ctx = Context(d, 32, 64)
    try:
        codes = np.array([[((3 * n + k) % 16) - 8 for k in range(K)] for n in range(N)])
        packed = inputs.pack_codes(codes)
        scales = inputs.uniform_f16(inputs.rng(9), 0.005, 0.02, (N, K // g))
        ctx.load_tensor(0, L.W4_T_LM_HEAD, 0, packed, scales)
        sv = f16v(scales)
        for k0 in range(0, K, 32):
            X = np.zeros((32, K))
            X[np.arange(32), k0 + np.arange(32)] = 1.0
            y = f16v(run(ctx, L.W4_T_LM_HEAD, inputs.f16_bits(X), N, gpu))
            ks = k0 + np.arange(32)
            want = (codes[:, ks] * sv[:, ks // g]).T
            assert np.array_equal(y, want.astype(np.float16).astype(np.float64)), k0
    finally:
        ctx.close()


def test_router_product_fp32(gpu):
    d = dataclasses.replace(inputs.TINY, n_layers=1)
    ctx = Context(d, 8, 64)
    try:
        w = inputs.w4_tensor(2, inputs.T_ROUTER, inputs.T_ROUTER_S, (), d.n_experts, d.hidden, d.group, (0,))
        ctx.load_tensor(0, L.W4_T_ROUTER, 0, w.packed, w.scales)
        x = inputs.normal_f16(inputs.rng(2, 7), (5, d.hidden))
        y = run(ctx, L.W4_T_ROUTER, x, d.n_experts, gpu, f32=True)
        ref = oracle.w4_gemm(x, w.packed, w.scales, d.group, out="f32")
        assert np.allclose(y, ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())
    finally:
        ctx.close()
