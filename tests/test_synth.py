"""Host side of the seeded input generator (its device twin is checked in the GPU tests)."""
import numpy as np

import k3x_synth as S


def test_splitmix64_published_outputs():
    # SplitMix64 seeded with 0: the first three outputs of the published generator
    w = S.stream_words(np.uint64(0), 0, 3)
    assert [int(v) for v in w] == [16294208416658607535, 7960286522194355700, 487617019471545679]


def test_packed_bytes_windowing_consistent():
    full = S.packed_bytes(5, 2, 7, S.W1_PACKED, 1000)
    for b0, n in ((0, 16), (3, 29), (500, 77), (992, 8)):
        assert np.array_equal(S.packed_bytes(5, 2, 7, S.W1_PACKED, n, b0=b0), full[b0:b0 + n])


def test_scale_bytes_windowing_and_range():
    full = S.scale_bytes(5, 1, 3, S.W2_SCALE, 4000)
    assert full.min() == 118 and full.max() == 130
    counts = np.bincount(full - 118, minlength=13)
    assert counts.min() > 4000 / 13 * 0.7
    for s0, n in ((1, 3), (7, 100), (3999, 1)):
        assert np.array_equal(S.scale_bytes(5, 1, 3, S.W2_SCALE, n, s0=s0), full[s0:s0 + n])


def test_nibbles_uniform():
    b = S.packed_bytes(9, 0, 0, S.W3_PACKED, 1 << 16)
    lo = np.bincount(b & 15, minlength=16)
    hi = np.bincount(b >> 4, minlength=16)
    assert lo.min() > 0.9 * 4096 and hi.min() > 0.9 * 4096


def test_streams_differ_between_tensors_and_experts():
    a = S.packed_bytes(1, 0, 0, S.W1_PACKED, 64)
    assert not np.array_equal(a, S.packed_bytes(1, 0, 1, S.W1_PACKED, 64))
    assert not np.array_equal(a, S.packed_bytes(1, 0, 0, S.W3_PACKED, 64))
    assert not np.array_equal(a, S.packed_bytes(1, 1, 0, S.W1_PACKED, 64))


def test_uniform_routing_properties():
    idx, gates = S.uniform_routing(3, 64, 896, 16)
    assert idx.shape == (64, 16) and gates.dtype == np.float32
    for t in range(64):
        assert len(set(idx[t].tolist())) == 16
    assert np.all(np.abs(gates.sum(axis=1, dtype=np.float64) - 1.0) < 1e-5)


def test_bf16_input_rounding():
    v = np.array([1.0, -2.5, 1.00390625, 3.14159], dtype=np.float32)
    b = S.f32_to_bf16_bits(v)
    assert b[0] == 0x3F80 and b[1] == 0xC020 and b[2] == 0x3F80  # tie to even
    assert abs(S.bf16_bits_to_f32(b[3]) - 3.14159) < 0.02


def test_zipf_bias_is_skewed():
    w = S.WORKLOADS[3]
    b = S.zipf_bias(w.seed, w.E)
    assert b.dtype == np.float32 and b.shape == (896,)
    assert b.max() - b.min() > 0.3
