"""The seeded input generator: published SplitMix64 outputs, determinism,
independence of row ranges, the canonical int4 storage format, and the
shape of the continuous-batching schedules."""
import numpy as np

from int4_w4a16_group_amd import inputs


def test_splitmix64_published_sequence():
    # reference outputs of splitmix64 seeded with 1234567 (Vigna's splitmix64.c)
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    got = inputs.splitmix_bytes(1234567, 40).view(np.uint64)
    assert [int(v) for v in got] == want


def test_splitmix_ranges_regenerate_independently():
    key = inputs.splitmix_key(0, 5, 7)
    full = inputs.splitmix_bytes(key, 10_000_000)
    part = inputs.splitmix_bytes(key, 4096, start=8 * 123_457)
    assert np.array_equal(part, full[8 * 123_457: 8 * 123_457 + 4096])
    assert np.array_equal(full, inputs.splitmix_bytes(key, 10_000_000, threads=1))


def test_int4_codes_uniform_and_pack_roundtrip():
    w = inputs.w4_tensor(0, inputs.T_QKV, inputs.T_QKV_S, (), 512, 2048, 128)
    c = inputs.unpack_codes(w.packed)
    assert c.min() == -8 and c.max() == 7
    counts = np.bincount(c.ravel() + 8, minlength=16)
    assert np.all(np.abs(counts / c.size - 1 / 16) < 0.002)
    assert np.array_equal(inputs.pack_codes(c), w.packed)
    s = w.scales.view(np.float16).astype(np.float64)
    assert s.min() >= 0.00499 and s.max() <= 0.02001


def test_generator_deterministic():
    a = inputs.make_layer(inputs.TINY, 0, 0)
    b = inputs.make_layer(inputs.TINY, 0, 0)
    c = inputs.make_layer(inputs.TINY, 1, 0)
    assert np.array_equal(a.gate.packed, b.gate.packed) and np.array_equal(a.qkv.scales, b.qkv.scales)
    assert not np.array_equal(a.gate.packed, c.gate.packed)


def test_skewed_routing_construction():
    for B in (1, 4, 8, 32):
        lg, (shared, private) = inputs.moe_logits(0, B, 128, "skewed")
        for b in range(B):
            top = set(np.argsort(-lg[b])[:8])
            assert top == set(shared) | set(private[b])
        assert len(set(private.ravel())) == 2 * B


def test_ragged_schedule_changes_batch_often():
    per_step, info = inputs.ragged_schedule(0, 200, 16, 0.25, 2048, 16, 512)
    sizes = [len(a) for a in per_step]
    assert min(sizes) >= 1 and max(sizes) <= 16
    changes = sum(1 for i in range(1, len(sizes)) if sizes[i] != sizes[i - 1])
    assert changes >= 10


def test_zero_mean_codes():
    w = inputs.w4_tensor(0, inputs.T_GATE, inputs.T_GATE_S, (), 256, 2048, 128, codes="zero_mean")
    c = inputs.unpack_codes(w.packed)
    assert c.min() == -7 and c.max() == 7
    counts = np.bincount(c.ravel() + 8, minlength=16)
    assert counts[0] == 0
    assert abs(c.mean()) < 0.01 and abs(counts[8] / c.size - 2 / 16) < 0.002
    u = inputs.w4_tensor(0, inputs.T_GATE, inputs.T_GATE_S, (), 256, 2048, 128)
    # same draw: only the -8 codes differ
    cu = inputs.unpack_codes(u.packed)
    assert np.array_equal(np.where(cu == -8, 0, cu), c)
