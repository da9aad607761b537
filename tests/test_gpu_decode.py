"""Decoder layer and whole decode step on the GPU against the oracle.

Layer: the tiny single MoE layer (hidden 256, 4 q / 2 kv heads x 64, 8 experts
top-2, intermediate 128, group 32), B=4 in an 8-slot x 128 arena at ragged
positions {3, 17, 40, 64}, slots reached through alloc/release.
Step: a small multi-layer model with vocabulary, several greedy steps with
the oracle's token fed to both sides (teacher forcing at near-ties), then the
batching invariants: batch vs alone, row order, slot id, stale (NaN) arena,
B x step(1) == step(B), and one launch sequence with no host sync per step.

Routing: the oracle is always run with the GPU's expert ids (its forced-routing
input), after checking that those ids are a top-k of the oracle's own router
logits up to the tolerance (exactly its top-k unless the k-th and (k+1)-th
logits are within it).  A near-tie therefore never ends a comparison."""
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


def near_tie(v, k, tol=TOL):
    s = np.sort(np.asarray(v, dtype=np.float64))[::-1]
    return s[k - 1] - s[k] <= tol * np.abs(s).max()


# ------------------------------------------------------------------ tiny layer
def test_tiny_layer_two_steps(gpu):
    case = inputs.tiny_layer_case(0)
    d = case["desc"]
    mw = inputs.make_model(d, 0, with_vocab=False)
    ctx = Context(d, case["n_slots"], case["cap"])
    om = oracle.Model(mw)
    oa = oracle.Arena(d, case["n_slots"], case["cap"])
    try:
        ctx.load_model(mw)
        # put the 4 streams in the seeded slots: fill every slot, free the chosen ones, re-join
        for _ in range(case["n_slots"]):
            L.w4_slot_alloc(ctx.ctx, 0, 1)
        for s in case["slots"]:
            ctx.release(int(s))
        slots = []
        for b in range(4):
            k, v = case["kv"][b]
            s = ctx.join(int(case["positions"][b]), 8, k, v)
            slots.append(s)
            oa.seed(s, k, v)
        assert sorted(slots) == sorted(int(s) for s in case["slots"])
        h = case["x"].copy()
        hd = to_dev(h, gpu)
        for step in range(2):
            pos = [ctx.position(s) for s in slots]
            ids = torch.empty((4, d.top_k), dtype=torch.int32, device=gpu)
            L.w4_layer_step(ctx.ctx, 0, slots, hd, ids, ctx.stream)
            gh, gids = to_host(hd), to_host(ids)
            rh, rids, rlg = oracle.layer_step(om, oa, 0, slots, pos, h, force=gids)
            for b in range(4):
                assert route_ok(gids[b], rlg[b], TOL), f"routing differs beyond a near-tie at step {step} row {b}"
            assert_normwise(f16v(gh), f16v(rh), TOL, f"layer step {step}")
            L.w4_slots_advance(ctx.ctx, slots)
            h = rh
            hd = to_dev(h, gpu)
    finally:
        ctx.close()


# Router geometries beyond the tiny and full models: the router runs one
# work-group per (row, 16-expert tile), each wave taking 128-column chunks
# w, w + 16, ...  H = 4096 gives two chunks per wave, 40 experts three tiles
# (the last one partial), g = 64 two scale groups per chunk; H = 1024 leaves
# half the waves without a chunk, 24 experts give two tiles.
ROUTER_SHAPES = {
    "h4096_e40_g64": dataclasses.replace(inputs.TINY, hidden=4096, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                                n_experts=40, top_k=4, moe_inter=256, group=64),
    "h1024_e24_g128": dataclasses.replace(inputs.TINY, hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=64,
                                                 n_experts=24, top_k=3, moe_inter=128, group=128),
}


@pytest.mark.parametrize("name", list(ROUTER_SHAPES))
def test_layer_router_geometries(gpu, name):
    d = ROUTER_SHAPES[name]
    positions = [1, 9, 30, 64, 100]
    B, n_slots, cap = len(positions), 8, 128
    mw = inputs.make_model(d, 3, with_vocab=False)
    ctx = Context(d, n_slots, cap)
    om = oracle.Model(mw)
    oa = oracle.Arena(d, n_slots, cap)
    try:
        ctx.load_model(mw)
        slots = []
        for b, p in enumerate(positions):
            k, v = inputs.prefix_kv(3, b, d.n_layers, p, d.n_kv_heads, d.head_dim)
            s = ctx.join(p, 4, k, v)
            oa.seed(s, k, v)
            slots.append(s)
        h = inputs.normal_f16(inputs.rng(3, inputs.T_X, d.hidden), (B, d.hidden))
        hd = to_dev(h, gpu)
        ids = torch.empty((B, d.top_k), dtype=torch.int32, device=gpu)
        L.w4_layer_step(ctx.ctx, 0, slots, hd, ids, ctx.stream)
        gh, gids = to_host(hd), to_host(ids)
        rh, rids, rlg = oracle.layer_step(om, oa, 0, slots, positions, h, force=gids)
        for b in range(B):
            assert route_ok(gids[b], rlg[b], TOL), f"{name}: routing differs beyond a near-tie at row {b}"
        assert_normwise(f16v(gh), f16v(rh), TOL, name)
    finally:
        ctx.close()


# The output projection at K = 4096 above 16 rows runs as two work-groups per
# tile (the second continues the first's in-order sum); 32 query heads x 128
# give K = 4096, B = 20 rows a 32-row tile, and g = 32 / 64 the scale groups
# the full model does not use.
@pytest.mark.parametrize("g", [32, 64])
def test_layer_split_output_projection(gpu, g):
    d = dataclasses.replace(inputs.TINY, hidden=512, n_q_heads=32, n_kv_heads=4, head_dim=128, n_experts=8,
                            top_k=2, moe_inter=128, group=g)
    B, n_slots, cap = 20, 24, 128
    positions = [(7 * b + 3) % 120 for b in range(B)]
    mw = inputs.make_model(d, 5, with_vocab=False)
    ctx = Context(d, n_slots, cap)
    om = oracle.Model(mw)
    oa = oracle.Arena(d, n_slots, cap)
    try:
        ctx.load_model(mw)
        slots = []
        for b, p in enumerate(positions):
            k, v = inputs.prefix_kv(5, b, d.n_layers, p, d.n_kv_heads, d.head_dim)
            s = ctx.join(p, 4, k, v)
            if p:
                oa.seed(s, k, v)
            slots.append(s)
        h = inputs.normal_f16(inputs.rng(5, inputs.T_X, g), (B, d.hidden))
        hd = to_dev(h, gpu)
        ids = torch.empty((B, d.top_k), dtype=torch.int32, device=gpu)
        L.w4_layer_step(ctx.ctx, 0, slots, hd, ids, ctx.stream)
        gh, gids = to_host(hd), to_host(ids)
        rh, rids, rlg = oracle.layer_step(om, oa, 0, slots, positions, h, force=gids)
        for b in range(B):
            assert route_ok(gids[b], rlg[b], TOL), f"g={g}: routing differs beyond a near-tie at row {b}"
        assert_normwise(f16v(gh), f16v(rh), TOL, f"g={g}")
    finally:
        ctx.close()


# ------------------------------------------------------------------ whole step
SMALL = dataclasses.replace(inputs.TINY, n_layers=3, vocab=500, top_k=2)


class Run:
    """A context plus the oracle mirror of the same streams."""

    def __init__(self, gpu, mw, n_slots=8, cap=256, poison=False):
        self.d = mw.desc
        self.ctx = Context(self.d, n_slots, cap)
        if poison:
            self.ctx.arena.view(torch.int16).fill_(0x7E00)
        self.ctx.load_model(mw)
        self.gpu = gpu

    def join(self, sid, plen, seed=0):
        k, v = inputs.prefix_kv(seed, sid, self.d.n_layers, plen, self.d.n_kv_heads, self.d.head_dim)
        return self.ctx.join(plen, 64, k, v), (k, v)

    def step(self, slots, tokens):
        B = len(slots)
        logits = empty_f16((B, self.d.vocab), self.gpu)
        nxt = torch.empty(B, dtype=torch.int32, device=self.gpu)
        ids = torch.empty((self.d.n_layers, B, self.d.top_k), dtype=torch.int32, device=self.gpu)
        tok = torch.tensor(np.asarray(tokens, np.int32), device=self.gpu)
        L.w4_decode_step(self.ctx.ctx, slots, tok, logits, nxt, ids, self.ctx.stream)
        return to_host(logits), to_host(nxt), to_host(ids)


@pytest.fixture(scope="module")
def small_model():
    return inputs.make_model(SMALL, 7)


def test_decode_steps_vs_oracle(gpu, small_model):
    mw = small_model
    run = Run(gpu, mw)
    om = oracle.Model(mw)
    oa = oracle.Arena(SMALL, 8, 256)
    prompts = [0, 5, 33, 100, 64]
    slots = []
    for sid, p in enumerate(prompts):
        s, (k, v) = run.join(sid, p)
        if p:
            oa.seed(s, k, v)
        slots.append(s)
    tokens = [inputs.first_token(0, sid, SMALL.vocab) for sid in range(len(prompts))]
    try:
        for step in range(6):
            pos = [run.ctx.position(s) for s in slots]
            lg, nxt, ids = run.step(slots, tokens)
            # the oracle replays the GPU's routing of every layer (accepted below)
            rl, rn, rids, rr = oracle.decode_step(om, oa, slots, pos, tokens, want_router=True, force=ids)
            for b in range(len(slots)):
                for l in range(SMALL.n_layers):
                    assert route_ok(ids[l, b], rr[l, b], TOL), f"routing differs beyond a near-tie: " \
                                                               f"layer {l} row {b} step {step}"
                assert_normwise(f16v(lg[b]), f16v(rl[b]), TOL, f"logits row {b} step {step}")
                if not near_tie(f16v(rl[b]), 1):
                    assert nxt[b] == rn[b]
                assert nxt[b] == int(np.argmax(f16v(lg[b])))
            tokens = [int(t) for t in rn]                      # the oracle's token goes to both
    finally:
        run.ctx.close()


def _fresh(gpu, mw, prompts, order=None, poison=False, slot_shift=0):
    run = Run(gpu, mw, poison=poison)
    for _ in range(slot_shift):
        L.w4_slot_alloc(run.ctx.ctx, 0, 1)
    slots = [run.join(sid, p)[0] for sid, p in enumerate(prompts)]
    return run, slots


def test_batch_invariants_bitwise(gpu, small_model):
    mw = small_model
    prompts = [3, 40, 0, 77]
    tokens = [11, 499, 0, 250]
    ref_run, slots = _fresh(gpu, mw, prompts)
    ref = [ref_run.step(slots, tokens)[0] for _ in range(3)]      # three steps, B = 4
    launches, syncs = L.w4_last_step_counts(ref_run.ctx.ctx)
    # embedding; per layer: q/k/v, attention (rotary, append and split combine included), o + residual,
    # router (norm, product, top-k, bucketing), gate/up, down, combine; output projection; argmax
    assert syncs == 0 and launches == 1 + SMALL.n_layers * 7 + 2
    ref_run.ctx.close()
    # I7: each stream stepped alone (B = 1), in separate calls, gives the same bits
    run, slots = _fresh(gpu, mw, prompts)
    for st in range(3):
        for b in range(4):
            lg, _, _ = run.step([slots[b]], [tokens[b]])
            assert np.array_equal(lg[0], ref[st][b]), (st, b)
    run.ctx.close()
    # I5 row order, I2 slot ids, I3 stale NaN arena
    perm = [2, 0, 3, 1]
    run, slots = _fresh(gpu, mw, prompts, poison=True, slot_shift=3)
    assert slots[0] == 3
    for st in range(3):
        lg, _, _ = run.step([slots[i] for i in perm], [tokens[i] for i in perm])
        for j, i in enumerate(perm):
            assert np.array_equal(lg[j], ref[st][i]), (st, i)
    run.ctx.close()


def test_ragged_join_finish_matches_solo(gpu, small_model):
    """Streams join and finish at different steps, freed slots are reused; every
    row of every composition equals that stream decoded alone."""
    mw = small_model
    # three slots: streams 3 and 4 join into the slots that 0 and 2 free
    sched = {0: [(0, 9)], 1: [(1, 30)], 3: [(2, 0)], 5: [(3, 12)], 6: [(4, 50)]}
    finish = {0: 4, 1: 7, 2: 5, 3: 8, 4: 9}
    run = Run(gpu, mw, n_slots=3)
    active, slot_of, history, freed, reused = [], {}, {}, set(), 0
    for step in range(10):
        for sid, p in sched.get(step, []):
            assert len(active) < 3, f"schedule joins stream {sid} into a full context"
            s, _ = run.join(sid, p)
            reused += s in freed
            slot_of[sid] = s
            active.append(sid)
            history[sid] = []
        if not active:
            continue
        toks = [(17 * sid + len(history[sid])) % SMALL.vocab for sid in active]
        lg, _, _ = run.step([slot_of[s] for s in active], toks)
        for j, sid in enumerate(active):
            history[sid].append(lg[j])
        for sid in list(active):
            if finish[sid] == step:
                run.ctx.release(slot_of[sid])
                freed.add(slot_of[sid])
                active.remove(sid)
    run.ctx.close()
    assert sorted(history) == [0, 1, 2, 3, 4] and reused == 2
    for sid, rows in history.items():
        prompt = dict(p for v in sched.values() for p in v)[sid]
        solo_run = Run(gpu, mw, n_slots=1)
        s, _ = solo_run.join(sid, prompt)
        for t, row in enumerate(rows):
            lg, _, _ = solo_run.step([s], [(17 * sid + t) % SMALL.vocab])
            assert np.array_equal(lg[0], row), (sid, t)
        solo_run.ctx.close()
