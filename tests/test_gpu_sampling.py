"""Non-greedy sampling on the GPU (temperature / top-k / top-p with a
counter-based draw per slot), through the C ABI.  Each sampled id is checked
against the oracle's sampler applied to the GPU's own logits row (so only
the sampler is under test): equal, except where the float64 restatement
puts the draw within 1e-5 of a boundary of the cumulative weights (either id
is then a correct sample).  A stream's sampled tokens and logits are the
same alone, in a batch, in any row order, and next to greedy rows."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from int4_w4a16_group_amd import _lib as L
from int4_w4a16_group_amd import inputs
from int4_w4a16_group_amd.engine import Context
from tests.gpu_util import empty_f16, to_host
from tests.test_oracle_sampling import ref_sample
from tests.util import f16v

pytestmark = pytest.mark.gpu
SMALL = dataclasses.replace(inputs.TINY, n_layers=3, vocab=500, top_k=2)
# (seed, temperature, top_k, top_p); temperature 0 is greedy
SETTINGS = [(11, 0.0, 1, 1.0), (12, 1.0, 64, 1.0), (13, 0.7, 20, 0.9), (2**63 + 5, 1.6, 5, 0.6)]


def check_sample(row_bits, got, T, k, p, seed, pos):
    want = oracle.sample(row_bits, T, k, p, seed, pos)
    if got != want:
        _, gap = ref_sample(row_bits, T, k, p, oracle.draw(seed, pos))
        assert gap < 1e-5, f"sampled {got}, oracle {want} (T={T} k={k} p={p} seed={seed} pos={pos})"


def run(ctx, gpu, slots, tokens):
    B = len(slots)
    lg = empty_f16((B, SMALL.vocab), gpu)
    nx = torch.empty(B, dtype=torch.int32, device=gpu)
    L.w4_decode_step(ctx.ctx, slots, torch.tensor(np.asarray(tokens, np.int32), device=gpu), lg, nx, None,
                     ctx.stream)
    return to_host(lg), to_host(nx)


def make(gpu, mw, n_slots=8):
    ctx = Context(SMALL, n_slots, 128)
    ctx.load_model(mw)
    return ctx


def join(ctx, sid, setting):
    p = 5 * sid + 3
    k, v = inputs.prefix_kv(9, sid, SMALL.n_layers, p, SMALL.n_kv_heads, SMALL.head_dim)
    s = ctx.join(p, 32, k, v)
    L.w4_slot_set_sampling(ctx.ctx, s, *setting)
    return s


def test_sampled_tokens_vs_oracle_and_batch_invariance(gpu):
    mw = inputs.make_model(SMALL, 8)
    n = len(SETTINGS)
    steps = 12
    ctx = make(gpu, mw)
    try:
        slots = [join(ctx, i, SETTINGS[i]) for i in range(n)]
        toks = [inputs.first_token(9, i, SMALL.vocab) for i in range(n)]
        hist_lg, hist_nx, fed = [], [], []
        for step in range(steps):
            pos = [ctx.position(s) for s in slots]
            lg, nx = run(ctx, gpu, slots, toks)
            for b in range(n):
                seed, T, k, p = SETTINGS[b]
                if T == 0:
                    assert nx[b] == int(np.argmax(f16v(lg[b])))
                check_sample(lg[b], int(nx[b]), T, k, p, seed, pos[b])
            hist_lg.append(lg)
            hist_nx.append(nx)
            fed.append(list(toks))
            toks = [int(t) for t in nx]
        sampled = {b for b in range(n) if SETTINGS[b][1] > 0 and len({int(h[b]) for h in hist_nx}) > 1}
        assert len(sampled) >= 2, "sampled streams should not all repeat one token"
    finally:
        ctx.close()
    # each stream alone, then all in reverse order on a fresh context: same bits
    for b in range(n):
        solo = make(gpu, mw, 1)
        try:
            s = join(solo, b, SETTINGS[b])
            for step in range(steps):
                lg, nx = run(solo, gpu, [s], [fed[step][b]])
                assert np.array_equal(lg[0], hist_lg[step][b]) and nx[0] == hist_nx[step][b], (b, step)
        finally:
            solo.close()
    rev = make(gpu, mw)
    try:
        for _ in range(3):                                     # other slot ids
            L.w4_slot_alloc(rev.ctx, 0, 1)
        order = list(range(n))[::-1]
        slots = {b: join(rev, b, SETTINGS[b]) for b in order}
        for step in range(steps):
            lg, nx = run(rev, gpu, [slots[b] for b in order], [fed[step][b] for b in order])
            for j, b in enumerate(order):
                assert np.array_equal(lg[j], hist_lg[step][b]) and nx[j] == hist_nx[step][b], (b, step)
    finally:
        rev.close()


def test_sampling_full_vocab_with_ties_at_the_cut(gpu):
    """Vocabulary 151936: top-k candidates found by the histogram passes, with
    ties at the k-th logit resolved to the lowest ids, over many draws."""
    d = dataclasses.replace(inputs.FULL, n_layers=1, n_experts=8, top_k=2, moe_inter=128)
    mw = inputs.make_model(d, 2, codes="zero_mean")
    for lw in mw.layers:
        lw.o.packed[:] = 0
        lw.down.packed[:] = 0
    # output projection zero except 20 random rows and 3 copies of one more: every
    # other logit is 0, so for most k the cut falls inside a tie of about 151900 ids
    # at 0, which must resolve to the lowest ids
    gq = inputs.rng(2, 55)
    lm = mw.lm_head
    keep = lm.packed.copy()
    lm.packed[:] = 0
    for i in gq.choice(d.vocab, 20, replace=False):
        lm.packed[i] = keep[i]
    q = gq.integers(-7, 8, size=(1, d.hidden))
    for i in (151000, 40, 99999):
        lm.packed[i] = inputs.pack_codes(q)[0]
        lm.scales[i] = lm.scales[7]
    ctx = Context(d, 32, 64)
    try:
        ctx.load_model(mw)
        B = 24
        settings = [(1000 + b, [0.6, 1.0, 2.0][b % 3], [3, 17, 64][b % 3], [1.0, 0.8, 0.95][b % 3]) for b in range(B)]
        slots = []
        for b in range(B):
            s = ctx.join(0, 4)
            L.w4_slot_set_sampling(ctx.ctx, s, *settings[b])
            slots.append(s)
        g = inputs.rng(2, inputs.T_TOKENS, 5)
        toks = [int(t) for t in g.integers(0, d.vocab, B)]
        for step in range(3):
            lg = empty_f16((B, d.vocab), gpu)
            nx = torch.empty(B, dtype=torch.int32, device=gpu)
            pos = [ctx.position(s) for s in slots]
            L.w4_decode_step(ctx.ctx, slots, torch.tensor(toks, dtype=torch.int32, device=gpu), lg, nx, None,
                             ctx.stream)
            lg, nx = to_host(lg), to_host(nx)
            for b in range(B):
                check_sample(lg[b], int(nx[b]), settings[b][1], settings[b][2], settings[b][3], settings[b][0],
                             pos[b])
            toks = [int(t) for t in nx]
    finally:
        ctx.close()
