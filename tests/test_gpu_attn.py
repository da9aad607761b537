"""Slot-indexed GQA decode attention on the GPU (32 q / 4 kv heads, head_dim
128, 16 slots x 4096-token cap) along a 200-step continuous-batching schedule:
streams join with seeded prompts, decode one token per step, finish, and
their slots are reused.  Every step is compared with the oracle, which keeps
its own KV store; a stream's output must not depend on the batch."""
import dataclasses

import numpy as np
import pytest

import oracle
from int4_w4a16_group_amd import _lib as L
from int4_w4a16_group_amd import inputs
from int4_w4a16_group_amd.engine import Context
from tests.gpu_util import empty_f16, to_dev, to_host
from tests.util import assert_normwise, f16v

pytestmark = pytest.mark.gpu
TOL = 2e-3
ATT = dataclasses.replace(inputs.FULL, n_layers=1, n_experts=8, top_k=2, moe_inter=128, vocab=16)


def attn(ctx, slots, q, k, v, dev):
    B = len(slots)
    o = empty_f16((B, ATT.n_q_heads, ATT.head_dim), dev)
    L.w4_attn_decode(ctx.ctx, 0, slots, to_dev(q, dev), to_dev(k, dev), to_dev(v, dev), o, ctx.stream)
    return to_host(o)


def test_ragged_schedule_200_steps(gpu):
    seed, S, cap = 0, 16, 4096
    per_step, info = inputs.ragged_schedule(seed, 200, S, 0.25, 2048, 16, 512)
    sizes = [len(a) for a in per_step]
    assert max(sizes) == S and min(sizes) == 1
    ctx = Context(ATT, S, cap)
    om = oracle.Model(inputs.ModelWeights(ATT, [inputs.make_layer(ATT, 0, 0)], None, None, None))
    oa = oracle.Arena(ATT, S, cap)
    slot_of, released, reused = {}, set(), 0
    try:
        for step, active in enumerate(per_step):
            for sid in active:
                if sid not in slot_of:
                    plen, life, _ = info[sid]
                    k, v = inputs.prefix_kv(seed, sid, 1, plen, ATT.n_kv_heads, ATT.head_dim)
                    s = ctx.join(plen, life, k, v)
                    reused += s in released
                    slot_of[sid] = s
                    oa.seed(s, k, v)
            slots = [slot_of[sid] for sid in active]
            pos = [ctx.position(s) for s in slots]
            q, kn, vn = inputs.attn_step_inputs(seed, step, len(slots), ATT.n_q_heads, ATT.n_kv_heads, ATT.head_dim)
            o = attn(ctx, slots, q, kn, vn, gpu)
            ro = oracle.attn_step(om, oa, 0, slots, pos, q, kn, vn)
            assert_normwise(f16v(o).reshape(len(slots), -1), f16v(ro).reshape(len(slots), -1), TOL, f"step {step}")
            if step % 50 == 7:                                # each row alone gives the same bits
                for b, s in enumerate(slots):
                    o1 = attn(ctx, [s], q[b:b + 1], kn[b:b + 1], vn[b:b + 1], gpu)
                    assert np.array_equal(o1[0], o[b])
            L.w4_slots_advance(ctx.ctx, slots)
            nxt = per_step[step + 1] if step + 1 < len(per_step) else []
            for sid in active:
                if sid not in nxt:
                    ctx.release(slot_of[sid])
                    released.add(slot_of[sid])
        assert reused > 0, "schedule never reused a slot"
    finally:
        ctx.close()


def test_single_position_and_poisoned_tail(gpu):
    """p = 0: output equals v_new exactly; stale arena contents (NaN) beyond p never leak."""
    import torch
    ctx = Context(ATT, 4, 128)
    try:
        ctx.arena.view(torch.int16).fill_(0x7E00)             # fp16 NaN everywhere
        s = ctx.join(0, 10)
        q, k, v = inputs.attn_step_inputs(3, 0, 1, ATT.n_q_heads, ATT.n_kv_heads, ATT.head_dim)
        o = attn(ctx, [s], q, k, v, gpu)
        G = ATT.n_q_heads // ATT.n_kv_heads
        for h in range(ATT.n_q_heads):
            assert np.array_equal(o[0, h], v[0, h // G])
        L.w4_slots_advance(ctx.ctx, [s])
        q2, k2, v2 = inputs.attn_step_inputs(3, 1, 1, ATT.n_q_heads, ATT.n_kv_heads, ATT.head_dim)
        o2 = attn(ctx, [s], q2, k2, v2, gpu)
        assert np.all(np.isfinite(f16v(o2)))
    finally:
        ctx.close()
