"""Seeded input generator: pinned to SplitMix64's published outputs and to
the distributions it claims to draw."""
import numpy as np

import synth


def test_splitmix64_published_sequence():
    # SplitMix64 started from state 0 emits e220a8397b1dcdaf, 6e789e6aa1b965f4,
    # 06c45d188009454f (the widely reproduced first outputs of Vigna's
    # splitmix64.c); state k*gamma is counter k*gamma here.
    g = synth.GAMMA
    c = np.array([0, g, (2 * g) % (1 << 64)], dtype=np.uint64)
    z = synth.splitmix64(c)
    assert [int(v) for v in z] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_uniform_range_and_moments():
    u = synth.uniform(7, 200000)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.005
    assert abs(u.var() - 1 / 12) < 0.002
    # 24-bit grid
    assert np.all((u * 2 ** 24) == np.floor(u * 2 ** 24))


def test_normal_moments_and_start_offset():
    n = synth.normal(9, (100000,))
    assert abs(n.mean()) < 0.02 and abs(n.std() - 1) < 0.02
    assert np.abs(n).max() < 6.0
    part = synth.normal(9, (10,), start=500)
    assert np.array_equal(part, n[500:510])


def test_xavier_bound():
    w = synth.xavier(3, (64, 32), 32, 64)
    a = np.sqrt(6 / 96)
    assert np.abs(w).max() <= a and np.abs(w).max() > 0.95 * a


def test_bf16_round_to_nearest_even():
    # 1 + 2**-8 is exactly half-way between bf16 neighbours 1 and 1 + 2**-7 -> even (1.0)
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    got = synth.bf16_bits_to_f32(synth.bf16_bits_from_f32(x))
    assert list(got) == [1.0, 1.0 + 2 ** -6, -2.5, 1.0 + 2 ** -7]


def test_ids_and_mixed_draws():
    p = synth.prompt(0, 4096, 512)
    assert p.min() >= 0 and p.max() < 512
    assert len(np.unique(p)) > 450
    T = synth.mixed_context_lengths(1000)
    assert T.min() >= 8192 and T.max() < 131072
    # log-uniform: median near sqrt(8192 * 131072) = 32768
    assert 26000 < np.median(T) < 41000
    x = synth.mixed_draft_horizons(1000)
    assert set(np.unique(x)) == {16, 24, 32, 40}


def test_outlier_channels_distinct():
    o = synth.outlier_channels(128, 128)
    for row in o:
        assert len(set(row.tolist())) == 4 and row.min() >= 0 and row.max() < 128
