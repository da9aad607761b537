"""Edge cases of the decode step on the GPU, through the C ABI:

* greedy ties: equal fp16 logits in different argmax splits must give the
  lowest id (the oracle's rule);
* the full-vocabulary output projection (151936 x 2048) through the decode
  step's own operand layout and tile loop, against the oracle;
* an out-of-range token id is reported (sticky W4_E_INVALID), never read, and
  leaves the other rows untouched;
* the K/V a slot holds reads back bit for bit (seeded prefix and appended
  positions)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from int4_w4a16_group_amd import _lib as L
from int4_w4a16_group_amd import inputs
from int4_w4a16_group_amd.engine import Context
from tests.gpu_util import empty_f16, to_dev, to_host
from tests.util import assert_normwise, f16v

pytestmark = pytest.mark.gpu
TOL = 2e-3


def zero_layer_outputs(mw):
    """Output-projection and down codes zero: every layer adds exactly zero to
    the residual stream, so the final state is the embedding row on both sides."""
    for lw in mw.layers:
        lw.o.packed[:] = 0
        lw.down.packed[:] = 0


def decode(ctx, slots, tokens, dev, vocab):
    B = len(slots)
    lg = empty_f16((B, vocab), dev)
    nx = torch.empty(B, dtype=torch.int32, device=dev)
    L.w4_decode_step(ctx.ctx, slots, torch.tensor(np.asarray(tokens, np.int32), device=dev), lg, nx, None,
                     ctx.stream)
    return to_host(lg), to_host(nx)


@pytest.mark.parametrize("vocab", [500, 499])      # 16-byte scan and the element-wise scan
def test_greedy_ties_take_the_lowest_id(gpu, vocab):
    d = dataclasses.replace(inputs.TINY, n_layers=1, vocab=vocab, top_k=2)
    mw = inputs.make_model(d, 9)
    zero_layer_outputs(mw)
    # output projection: zero except three identical rows (ids 70, 3, 490, in
    # argmax splits 1, 0 and 7) and three exact negations of them (200, 9, 450):
    # every logit is exactly +L, -L or 0, so the greedy id is 3 when L > 0 and 9
    # when L < 0, each a tie across splits
    q = inputs.rng(9, 77).integers(-7, 8, size=(1, d.hidden))
    pos_ids, neg_ids = [70, 3, 490], [200, 9, 450]
    lm = mw.lm_head
    lm.packed[:] = 0
    s_row = lm.scales[5].copy()
    for i in pos_ids:
        lm.packed[i] = inputs.pack_codes(q)[0]
        lm.scales[i] = s_row
    for i in neg_ids:
        lm.packed[i] = inputs.pack_codes(-q)[0]
        lm.scales[i] = s_row
    ctx = Context(d, 8, 64)
    try:
        ctx.load_model(mw)
        tokens = [1, 17, 250, 333, 480, 64]
        slots = [ctx.join(0, 4) for _ in tokens]
        lg, nx = decode(ctx, slots, tokens, gpu, vocab)
        om, oa = oracle.Model(mw), oracle.Arena(d, 8, 64)
        rl, rn, _, _ = oracle.decode_step(om, oa, slots, [0] * len(tokens), tokens)
        signs = set()
        for b in range(len(tokens)):
            v = f16v(lg[b])
            assert np.array_equal(v[pos_ids], np.full(3, v[3])) and np.array_equal(v[neg_ids], -v[pos_ids])
            assert np.all(v[np.setdiff1d(np.arange(vocab), pos_ids + neg_ids)] == 0)
            want = 3 if v[3] > 0 else (9 if v[3] < 0 else 0)
            signs.add(np.sign(v[3]))
            assert nx[b] == want, (b, v[3], nx[b])
            assert rn[b] == (3 if f16v(rl[b])[3] > 0 else 9 if f16v(rl[b])[3] < 0 else 0)
        assert signs == {1.0, -1.0}, "the tokens should exercise both tie groups"
    finally:
        ctx.close()


def test_full_vocab_output_projection_in_the_decode_step(gpu):
    """The decode step's output projection reads the final normalised state as an
    activation panel and loops about 18 column tiles per work-group at vocab
    151936; checked against the oracle at B = 20 (32-row tiles) and B = 5."""
    d = dataclasses.replace(inputs.FULL, n_layers=1, n_experts=8, top_k=2, moe_inter=128)
    mw = inputs.make_model(d, 2, codes="zero_mean")
    zero_layer_outputs(mw)
    om = oracle.Model(mw)
    ctx = Context(d, 32, 64)
    try:
        ctx.load_model(mw)
        g = inputs.rng(2, inputs.T_TOKENS, 99)
        for B in (20, 5):
            tokens = [int(t) for t in g.integers(0, d.vocab, B)]
            slots = [ctx.join(0, 4) for _ in range(B)]
            lg, nx = decode(ctx, slots, tokens, gpu, d.vocab)
            rl, rn, _, _ = oracle.decode_step(om, oracle.Arena(d, 32, 64), slots, [0] * B, tokens)
            assert_normwise(f16v(lg), f16v(rl), TOL, f"full-vocab logits B={B}")
            o = f16v(rl)
            srt = np.sort(o, 1)
            gated = (srt[:, -1] - srt[:, -2]) > TOL * np.abs(o).max(1)
            assert np.all((nx == rn) | ~gated)
            assert np.all(nx == np.argmax(f16v(lg), 1))
            for s in slots:
                ctx.release(s)
    finally:
        ctx.close()


SMALL = dataclasses.replace(inputs.TINY, n_layers=2, vocab=500, top_k=2)


def test_invalid_token_is_reported_and_not_read(gpu):
    mw = inputs.make_model(SMALL, 7)
    ctx = Context(SMALL, 4, 64)
    ref = Context(SMALL, 4, 64)
    try:
        ctx.load_model(mw)
        ref.load_model(mw)
        a, b = ctx.join(0, 8), ctx.join(0, 8)
        ra, rb = ref.join(0, 8), ref.join(0, 8)
        lg, _ = decode(ctx, [a, b], [5, SMALL.vocab + 3], gpu, SMALL.vocab)   # row 1 out of range
        rlg, _ = decode(ref, [ra, rb], [5, 11], gpu, SMALL.vocab)
        assert np.array_equal(lg[0], rlg[0])                   # the other row is untouched
        with pytest.raises(L.W4Error) as e:
            L.w4_check_errors(ctx.ctx)
        assert e.value.status == L.W4_E_INVALID
        assert L.w4_check_errors(ctx.ctx) == L.W4_OK           # reported once
        # a negative id: the next enqueueing call reports it and does nothing
        decode(ctx, [a, b], [-1, 7], gpu, SMALL.vocab)
        torch.cuda.synchronize()
        pa = ctx.position(a)
        with pytest.raises(L.W4Error) as e:
            decode(ctx, [a, b], [5, 7], gpu, SMALL.vocab)
        assert e.value.status == L.W4_E_INVALID and ctx.position(a) == pa
        decode(ctx, [a, b], [5, 7], gpu, SMALL.vocab)          # and the context goes on
        assert L.w4_check_errors(ctx.ctx) == L.W4_OK
    finally:
        ctx.close()
        ref.close()


def test_kv_readback_round_trip(gpu):
    d = dataclasses.replace(inputs.TINY, n_layers=2)
    ctx = Context(d, 4, 128)
    try:
        p = 70
        k, v = inputs.prefix_kv(4, 0, d.n_layers, p, d.n_kv_heads, d.head_dim)
        s = ctx.join(p, 8, k, v)
        rk, rv = ctx.read_kv(s)
        assert np.array_equal(rk, k) and np.array_equal(rv, v)
        q, kn, vn = inputs.attn_step_inputs(4, 0, 1, d.n_q_heads, d.n_kv_heads, d.head_dim)
        o = empty_f16((1, d.n_q_heads, d.head_dim), gpu)
        L.w4_attn_decode(ctx.ctx, 1, [s], to_dev(q, gpu), to_dev(kn, gpu), to_dev(vn, gpu), o, ctx.stream)
        L.w4_slots_advance(ctx.ctx, [s])
        rk, rv = ctx.read_kv(s)
        assert rk.shape == (d.n_layers, p + 1, d.n_kv_heads, d.head_dim)
        assert np.array_equal(rk[:, :p], k) and np.array_equal(rv[:, :p], v)
        assert np.array_equal(rk[1, p], kn[0]) and np.array_equal(rv[1, p], vn[0])
    finally:
        ctx.close()
