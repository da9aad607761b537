"""Seed-at-join prefill on the GPU through the C ABI: a joining stream's prompt
goes through the model (M = P row products, the slot's K/V written with
rotary keys, causal attention over the slot, one grouped expert product per
layer over the prompt's routed rows).  Checked against the oracle's prefill,
which runs the same tokens one by one through its decode step (the GPU's
expert ids replayed once each is accepted as a top-k of the oracle's router
logits within the tolerance): the K/V of every position and layer, the last
token's logits and next id, and the first decode step after the join.  A
prefill writes no other slot."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from int4_w4a16_group_amd import _lib as L
from int4_w4a16_group_amd import inputs
from int4_w4a16_group_amd.engine import Context
from tests.gpu_util import empty_f16, to_host
from tests.test_gpu_sampling import check_sample
from tests.util import assert_normwise, f16v, normwise_err, route_ok

pytestmark = pytest.mark.gpu
TOL = 2e-3
SMALL = dataclasses.replace(inputs.TINY, n_layers=3, vocab=500, top_k=2)


def gpu_prefill(ctx, gpu, tokens, max_new=8):
    d = ctx.desc
    P = len(tokens)
    lg = empty_f16((d.vocab,), gpu)
    nx = torch.empty(1, dtype=torch.int32, device=gpu)
    ids = torch.empty((d.n_layers, P, d.top_k), dtype=torch.int32, device=gpu)
    s = ctx.prefill(tokens, max_new, lg, nx, ids)
    return s, to_host(lg), int(to_host(nx)[0]), to_host(ids)


def check_prefill(ctx, gpu, mw, tokens, what):
    """GPU prefill of a new stream against the oracle; returns (slot, oracle model, oracle arena)."""
    d = ctx.desc
    P = len(tokens)
    s, lg, nx, ids = gpu_prefill(ctx, gpu, tokens)
    om = oracle.Model(mw)
    oa = oracle.Arena(d, 1, (P + 64) // 64 * 64)
    rl, rn, _, rr = oracle.prefill(om, oa, 0, tokens, force=ids, want_ids=True, want_router=True)
    assert ctx.position(s) == P
    k, v = ctx.read_kv(s)
    report = []
    for name, g, r in (("K", k, oa.k[:, 0, :P]), ("V", v, oa.v[:, 0, :P])):
        e = normwise_err(f16v(g).reshape(d.n_layers, P, -1), f16v(r).reshape(d.n_layers, P, -1))
        for l in range(d.n_layers):
            report.append(f"{name} layer {l}: worst {e[l].max():.2e} at {int(e[l].argmax())}")
    bad = []
    for l in range(d.n_layers):
        for t in range(P):
            if not route_ok(ids[l, t], rr[l, t], TOL):
                lg_ = rr[l, t].astype(np.float64)
                sel = lg_[ids[l, t]]
                rest = np.delete(lg_, ids[l, t])
                bad.append(f"layer {l} pos {t}: gpu {sorted(ids[l, t].tolist())} oracle top "
                           f"{sorted(np.argsort(-lg_, kind='stable')[:d.top_k].tolist())}; min selected "
                           f"{sel.min():.5f}, max other {rest.max():.5f}, tolerance {TOL * np.abs(lg_).max():.5f}")
    assert not bad, f"{what}: {len(bad)} routing choices beyond a near-tie: {bad[:4]}; {report}"
    for name, g, r in (("K", k, oa.k[:, 0, :P]), ("V", v, oa.v[:, 0, :P])):
        gg = f16v(g).reshape(d.n_layers * P, -1)
        rr_ = f16v(r).reshape(d.n_layers * P, -1)
        assert_normwise(gg, rr_, TOL, f"{what}: {name} ({report})")
    assert_normwise(f16v(lg), f16v(rl), TOL, f"{what}: last-token logits")
    o = f16v(rl)
    srt = np.sort(o)
    if srt[-1] - srt[-2] > TOL * np.abs(o).max():
        assert nx == rn, what
    assert nx == int(np.argmax(f16v(lg)))
    return s, om, oa


@pytest.fixture(scope="module")
def small(gpu):
    mw = inputs.make_model(SMALL, 12)
    ctx = Context(SMALL, 4, 256)
    ctx.load_model(mw)
    yield mw, ctx
    ctx.close()


@pytest.mark.parametrize("P", [1, 17, 64, 65, 130])
def test_prefill_small_model_vs_oracle(small, gpu, P):
    mw, ctx = small
    tokens = [int(t) for t in inputs.rng(12, inputs.T_TOKENS, P).integers(0, SMALL.vocab, P)]
    s, om, oa = check_prefill(ctx, gpu, mw, tokens, f"P={P}")
    try:
        # the first decode step after the join
        tok = 7
        lg = empty_f16((1, SMALL.vocab), gpu)
        nx = torch.empty(1, dtype=torch.int32, device=gpu)
        ids = torch.empty((SMALL.n_layers, 1, SMALL.top_k), dtype=torch.int32, device=gpu)
        L.w4_decode_step(ctx.ctx, [s], torch.tensor([tok], dtype=torch.int32, device=gpu), lg, nx, ids, ctx.stream)
        gids = to_host(ids)
        rl, rn, _, rr = oracle.decode_step(om, oa, [0], [P], [tok], want_router=True, force=gids)
        for l in range(SMALL.n_layers):
            assert route_ok(gids[l, 0], rr[l, 0], TOL)
        assert_normwise(f16v(to_host(lg)[0]), f16v(rl[0]), TOL, f"P={P}: decode step after the prefill")
    finally:
        ctx.release(s)


def test_prefill_three_layers_shared_bucketing(gpu):
    """A 700-token prompt on the three-layer model: 1400 routed pairs, so the
    bucketing runs as two work-groups sharing the pairs, and its row masks
    alternate between two buffers over the layers (each layer's launch clears
    the next one's).  Checked against the oracle like the shorter prompts."""
    mw = inputs.make_model(SMALL, 12)
    ctx = Context(SMALL, 2, 768)
    try:
        ctx.load_model(mw)
        P = 700
        tokens = [int(t) for t in inputs.rng(12, inputs.T_TOKENS, P).integers(0, SMALL.vocab, P)]
        s, _, _ = check_prefill(ctx, gpu, mw, tokens, f"P={P}, three layers")
        ctx.release(s)
    finally:
        ctx.close()


def test_prefill_leaves_other_slots_alone(small, gpu):
    """A stream decoding next to another stream's prefill: its K/V and its next
    decode step are bit-identical to the same stream with no neighbour."""
    mw, ctx = small
    k, v = inputs.prefix_kv(12, 0, SMALL.n_layers, 40, SMALL.n_kv_heads, SMALL.head_dim)
    a = ctx.join(40, 8, k, v)
    try:
        lg0 = empty_f16((1, SMALL.vocab), gpu)
        nx = torch.empty(1, dtype=torch.int32, device=gpu)
        ref_ctx = Context(SMALL, 4, 256)
        ref_ctx.load_model(mw)
        ra = ref_ctx.join(40, 8, k, v)
        L.w4_decode_step(ref_ctx.ctx, [ra], torch.tensor([3], dtype=torch.int32, device=gpu), lg0, nx, None,
                         ref_ctx.stream)
        ref = to_host(lg0)
        ref_ctx.close()
        b, _, _, _ = gpu_prefill(ctx, gpu, list(range(100, 190)))
        rk, rv = ctx.read_kv(a)
        assert np.array_equal(rk, k) and np.array_equal(rv, v)
        lg = empty_f16((1, SMALL.vocab), gpu)
        L.w4_decode_step(ctx.ctx, [a], torch.tensor([3], dtype=torch.int32, device=gpu), lg, nx, None, ctx.stream)
        assert np.array_equal(to_host(lg), ref)
        ctx.release(b)
    finally:
        ctx.release(a)


def test_prefill_sampled_first_token_and_invalid_ids(small, gpu):
    mw, ctx = small
    d = SMALL
    tokens = [int(t) for t in inputs.rng(13, 2).integers(0, d.vocab, 33)]
    s = L.w4_slot_alloc(ctx.ctx, len(tokens), 4)
    L.w4_slot_set_sampling(ctx.ctx, s, 99, 0.9, 30, 0.95)
    nbytes = L.w4_prefill_workspace_bytes(d, len(tokens), ctx.cap)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=gpu)
    lg = empty_f16((d.vocab,), gpu)
    nx = torch.empty(1, dtype=torch.int32, device=gpu)
    L.w4_slot_prefill(ctx.ctx, s, torch.tensor(tokens, dtype=torch.int32, device=gpu), ws, nbytes, lg, nx, None,
                      ctx.stream)
    check_sample(to_host(lg), int(to_host(nx)[0]), 0.9, 30, 0.95, 99, len(tokens) - 1)
    ctx.release(s)
    bad = list(tokens)
    bad[5] = d.vocab + 1
    s = L.w4_slot_alloc(ctx.ctx, len(bad), 4)
    L.w4_slot_prefill(ctx.ctx, s, torch.tensor(bad, dtype=torch.int32, device=gpu), ws, nbytes, None, None, None,
                      ctx.stream)
    with pytest.raises(L.W4Error) as e:
        L.w4_check_errors(ctx.ctx)
    assert e.value.status == L.W4_E_INVALID and "prefill" in str(e.value)
    ctx.release(s)


@pytest.mark.parametrize("P", [2048, 1957])
def test_prefill_full_geometry_longest_prompt(gpu, P):
    """Hidden 2048, 32q/4kv x 128, 128 experts top-8, intermediate 768, vocab
    151936, group 128, one layer; the longest prompt the prefill routing takes
    (2048 tokens: 16384 routed pairs, 128 + 1024 + 1 expert work units against a
    decode step's 289, 64 attention chunks, up to 8 splits) and a ragged one
    (1957 tokens: the last 128-row block of the q/k/v and output products holds
    37 rows, under both the 256- and the 128-column blocks).  One layer, so the
    comparison starts from exact inputs: through a second free-running layer
    this random model already amplifies rounding differences to about the
    tolerance (the reason full-size decode parity is checked layer by layer);
    the multi-layer prefill is checked on the three-layer model above."""
    d = dataclasses.replace(inputs.FULL, n_layers=1)
    mw = inputs.make_model(d, 4, codes="zero_mean")
    ctx = Context(d, 2, 2112)
    try:
        ctx.load_model(mw)
        tokens = [int(t) for t in inputs.rng(4, inputs.T_TOKENS, 1).integers(0, d.vocab, P)]
        s, _, _ = check_prefill(ctx, gpu, mw, tokens, f"full geometry P={P}")
        ctx.release(s)
    finally:
        ctx.close()
