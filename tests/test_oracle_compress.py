"""Compressor pins: hand-worked quantization and packing fixtures, closed-form
cases, brute-force code search, and token-drop selection on crafted inputs."""
import math
import os

import numpy as np
import pytest

from oracle.compress import (Quantized, pack_bits, quant_blob, quant_groups, quant_sizes, tokdrop,
                             tokdrop_scores, tokdrop_select, unpack_bits)

HERE = os.path.join(os.path.dirname(__file__), "golden")


def _kv(path):
    out = []
    for line in open(os.path.join(HERE, path)):
        if line.startswith("#") or not line.strip():
            continue
        out.append(dict(f.split("=") for f in line.split()))
    return out


def test_pack_bits_fixture():
    for row in _kv("pack_bits.txt"):
        b = int(row["bits"])
        codes = np.array([int(c) for c in row["codes"].split(",")], dtype=np.uint8)
        want = bytes(int(h, 16) for h in row["bytes"].split(","))
        assert pack_bits(codes, b).tobytes() == want
        assert np.array_equal(unpack_bits(np.frombuffer(want, np.uint8), b, len(codes)), codes)


def test_quant_group_fixture():
    for row in _kv("quant_group.txt"):
        b = int(row["bits"])
        x = np.array([float(v) for v in row["values"].split(",")], dtype=np.float32)
        codes, s, z = quant_groups(x[None], b)
        assert float(s[0]) == float(row["scale"])
        assert float(z[0]) == float(np.float32(float(row["zero"])))
        assert codes[0].tolist() == [int(c) for c in row["codes"].split(",")]


@pytest.mark.parametrize("b", [2, 3, 4])
def test_ramp_exact_codes(b):
    # zero and step exactly representable in fp16; x = zero + k * step hits codes 0..2^b-1
    step, zero = 0.25, -1.5
    k = np.arange(2 ** b)
    x = (zero + k * step).astype(np.float32)
    codes, s, z = quant_groups(x[None], b)
    assert float(s[0]) == step and float(z[0]) == zero
    assert codes[0].tolist() == k.tolist()


@pytest.mark.parametrize("b", [2, 3, 4])
def test_reconstruction_bound_and_brute_force(b):
    rng = np.random.default_rng(b)
    x = (rng.normal(size=(64, 128)) * rng.uniform(0.1, 20, size=(64, 1))).astype(np.float32)
    codes, s, z = quant_groups(x, b)
    s64, z64 = s.astype(np.float64)[:, None], z.astype(np.float64)[:, None]
    xhat = codes * s64 + z64
    # fp16 rounding of zero (<= half spacing of |mn|) plus half a step, plus the top-end fp16 scale error
    bound = s64 / 2 + np.abs(z64) * 2 ** -11 + (2 ** b - 1) * s64 * 2 ** -11 + 1e-7
    assert np.all(np.abs(x - xhat) <= bound + 1e-6)
    # brute force: the code is the nearest grid point (in float32 arithmetic) except exact ties
    grid = np.arange(2 ** b)
    t = (x.astype(np.float32) - z.astype(np.float32)[:, None]) / s.astype(np.float32)[:, None]
    dist = np.abs(t[..., None].astype(np.float64) - grid)
    best = dist.argmin(axis=-1)
    tie = np.isclose(np.sort(dist, axis=-1)[..., 0], np.sort(dist, axis=-1)[..., 1])
    assert np.all((best == codes) | tie)


def test_constant_group_scale_zero():
    x = np.full((1, 64), 3.140625, dtype=np.float32)
    codes, s, z = quant_groups(x, 3)
    assert float(s[0]) == 0.0 and np.all(codes == 0) and float(z[0]) == 3.140625


def test_quantized_layout_and_blob_sizes():
    rng = np.random.default_rng(5)
    L, H, T, D, G = 2, 3, 200, 128, 64
    K = rng.normal(size=(L, H, T, D)).astype(np.float32)
    V = rng.normal(size=(L, H, T, D)).astype(np.float32)
    q = Quantized(K, V, 3, G)
    assert q.Tq == 192 and q.kcodes.shape == (L, H, 192, D) and q.ks.shape == (L, H, 3, D)
    assert q.vs.shape == (L, H, 192, 2)
    # K groups run along tokens for one channel
    c, s, z = quant_groups(K[1, 2, 64:128, 5][None], 3)
    assert np.array_equal(q.kcodes[1, 2, 64:128, 5], c[0]) and q.ks[1, 2, 1, 5] == s[0]
    # V groups run along channels for one token
    c, s, z = quant_groups(V[0, 1, 7, 64:128][None], 3)
    assert np.array_equal(q.vcodes[0, 1, 7, 64:128], c[0]) and q.vs[0, 1, 7, 1] == s[0]
    blob = quant_blob(q, "fp32")
    sizes = quant_sizes(L, H, T, D, 3, G, 4)
    aligned = sum((n + 255) // 256 * 256 for n in sizes)
    assert len(blob) == aligned
    # first section: token rows of K codes, little-endian 3-bit stream over channels
    row = np.frombuffer(blob[: D * 3 // 8], np.uint8)
    assert np.array_equal(unpack_bits(row, 3, D), q.kcodes[0, 0, 0])


def test_tokdrop_keeps_everything_when_it_fits():
    T, D = 40, 8
    idx = tokdrop_select(np.zeros(T), T, keep_total=64, keep_recent=16)
    assert idx.tolist() == list(range(T))


def test_tokdrop_crafted_attention():
    """One-hot keys: the observation queries point at channel 0, so exactly the
    keys with a large channel-0 entry take (almost) all the attention."""
    T, D, G, W = 96, 8, 2, 4
    K = np.zeros((T, D))
    hot = [3, 17, 20, 41, 55]
    K[hot, 0] = 8.0
    q = np.zeros((G, W, D))
    q[:, :, 0] = 8.0
    s = tokdrop_scores(q, K, T - 16)
    idx = tokdrop_select(s, T, keep_total=16 + len(hot), keep_recent=16)
    assert idx.tolist() == hot + list(range(T - 16, T))


def test_tokdrop_topk_brute_force_and_ties():
    rng = np.random.default_rng(3)
    T, R, Kt = 300, 20, 80
    for trial in range(20):
        s = rng.integers(0, 6, size=T - R).astype(float)      # many ties
        idx = tokdrop_select(s, T, Kt, R)
        ranked = sorted(range(T - R), key=lambda t: (-s[t], t))
        want = sorted(ranked[: Kt - R]) + list(range(T - R, T))
        assert idx.tolist() == want


def test_tokdrop_scores_are_probabilities():
    rng = np.random.default_rng(4)
    T, D, G, W = 64, 8, 2, 4
    K = rng.normal(size=(T, D))
    q = rng.normal(size=(G, W, D))
    s = tokdrop_scores(q, K, T)           # all keys as candidates: each (h, i) row sums to 1
    assert abs(s.sum() - 1.0) < 1e-12


def test_tokdrop_gather():
    rng = np.random.default_rng(6)
    L, H, T, D, G, W = 1, 2, 64, 4, 2, 4
    K = rng.normal(size=(L, H, T, D))
    V = rng.normal(size=(L, H, T, D))
    q = rng.normal(size=(L, H * G, W, D))
    idx, Kk, Vk, _ = tokdrop(K, V, q, keep_total=24, keep_recent=8, group=G)
    assert idx.shape == (L, H, 24)
    for j in range(H):
        assert np.all(np.diff(idx[0, j]) > 0)
        assert np.array_equal(Kk[0, j], K[0, j, idx[0, j]])
        assert idx[0, j, -8:].tolist() == list(range(56, 64))


# ------------------------------------------------------------------ token drop by key norm
def test_keynorm_known_norms_and_shared_set():
    """Every head's key t has norm 1 + t mod 7 (in a different channel per head): the largest
    norms are known, ties go to the smaller position, and every head keeps the same set."""
    from oracle.compress import tokdrop_keynorm
    L, H, T, D = 2, 3, 40, 4
    K = np.zeros((L, H, T, D))
    for t in range(T):
        for j in range(H):
            K[:, j, t, j] = 1 + t % 7
    V = np.arange(L * H * T * D, dtype=float).reshape(L, H, T, D)
    idx, Kk, Vk, e = tokdrop_keynorm(K, V, keep_total=8)
    # norm 7 at t = 6, 13, 20, 27, 34 (five tokens), then norm 6 at t = 5, 12, 19, 26, 33: the
    # three smallest positions of those take the remaining places
    assert idx[0, 0].tolist() == [5, 6, 12, 13, 19, 20, 27, 34]
    assert all(idx[l, j].tolist() == idx[0, 0].tolist() for l in range(L) for j in range(H))
    assert np.array_equal(Vk[1, 2], V[1, 2, idx[1, 2]])
    assert np.allclose(e[0], 1 + np.arange(T) % 7)


def test_keynorm_mean_over_heads_decides():
    """Head 0 prefers token 0, head 1 prefers token 1; token 1's mean norm is larger."""
    from oracle.compress import keynorm_scores, tokdrop_keynorm
    K = np.zeros((1, 2, 3, 2))
    K[0, 0, 0] = [3.0, 4.0]     # norm 5
    K[0, 1, 0] = [0.0, 1.0]     # norm 1   -> mean 3
    K[0, 0, 1] = [0.0, 2.0]     # norm 2
    K[0, 1, 1] = [6.0, 0.0]     # norm 6   -> mean 4
    K[0, :, 2] = [1.0, 0.0]     #          -> mean 1
    assert keynorm_scores(K[0]).tolist() == [3.0, 4.0, 1.0]
    idx, _, _, _ = tokdrop_keynorm(K, K, keep_total=1)
    assert idx[0, 0].tolist() == [1] and idx[0, 1].tolist() == [1]


def test_keynorm_plain_loop_and_keep_all():
    from oracle.compress import keynorm_scores, tokdrop_keynorm
    rng = np.random.default_rng(5)
    K = rng.normal(size=(3, 17, 6))
    e = keynorm_scores(K)
    for t in range(17):
        norms = [math.sqrt(sum(K[j, t, d] ** 2 for d in range(6))) for j in range(3)]
        assert abs(e[t] - sum(norms) / 3) < 1e-12
    idx, _, _, _ = tokdrop_keynorm(K[None], K[None], keep_total=40)
    assert idx[0, 1].tolist() == list(range(17))
