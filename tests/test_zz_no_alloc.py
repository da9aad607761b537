"""The allocation-free routing entry point (w4_route_noalloc: no context, its
scratch in a static device array) against the context-based w4_route through
the C ABI: every output bit-identical on two calls in a row, the second with
fewer rows, and the routing ids equal to the oracle's top-k."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from int4_w4a16_group_amd import _lib as L
from int4_w4a16_group_amd import inputs
from int4_w4a16_group_amd.engine import Context
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu
DESC = dataclasses.replace(inputs.TINY, hidden=512, moe_inter=512, n_experts=128, top_k=8)


def outputs(B, E, k, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    return dict(ids=torch.full((B, k), -7, **i32), w=torch.full((B, k), -1.0, dtype=torch.float32, device=dev),
                counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
                ps=torch.full((B * k,), -7, **i32), pr=torch.full((B * k,), -7, **i32))


def test_route_noalloc_matches_context_route(gpu):
    E, k = DESC.n_experts, DESC.top_k
    ctx = Context(DESC, 32, 64)
    try:
        for call, B in enumerate((32, 5)):                 # two calls in a row, the second smaller
            logits, _ = inputs.moe_logits(40 + call, B, E, "disjoint")
            logits[0, 3] = logits[0, 100] = logits[0].max() + 1.0          # an exact tie: lower id first
            ld = to_dev(logits, gpu)
            a, b = outputs(B, E, k, gpu), outputs(B, E, k, gpu)
            L.w4_route(ctx.ctx, B, ld, a["ids"], a["w"], a["counts"], a["offsets"], a["ps"], a["pr"], ctx.stream)
            L.w4_route_noalloc(B, E, k, ld, b["ids"], b["w"], b["counts"], b["offsets"], b["ps"], b["pr"],
                               ctx.stream)
            for name in a:
                x, y = to_host(a[name]), to_host(b[name])
                assert np.array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                      y.view(np.uint32) if y.dtype == np.float32 else y), (call, name)
            rids, _ = oracle.topk_softmax(logits, k)
            assert np.array_equal(to_host(b["ids"]), rids)
            assert to_host(b["ids"])[0, 0] == 3 and to_host(b["ids"])[0, 1] == 100
    finally:
        ctx.close()


def test_route_noalloc_rejects_sizes_beyond_its_scratch(gpu):
    dev = gpu
    ld = torch.zeros((33, 128), dtype=torch.float32, device=dev)
    ids = torch.empty((33, 8), dtype=torch.int32, device=dev)
    w = torch.empty((33, 8), dtype=torch.float32, device=dev)
    for B, E, k in ((33, 128, 8), (4, 257, 8), (4, 128, 17)):
        with pytest.raises(L.W4Error) as e:
            L.w4_route_noalloc(B, E, k, ld, ids, w)
        assert e.value.status == L.W4_E_UNSUPPORTED and "w4_route_noalloc" in str(e.value)
    with pytest.raises(L.W4Error) as e:
        L.w4_route_noalloc(4, 128, 8, None, ids, w)
    assert e.value.status == L.W4_E_INVALID
