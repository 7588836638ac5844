"""Model pins: closed forms for RMSNorm and RoPE, and the cached greedy decode
against a brute-force no-cache recomputation."""
import math

import numpy as np
import pytest

import synth
from oracle import decode as D
from oracle.model import Weights, argmax, attend, rmsnorm, rope, sequence_logits
from oracle.rounding import to_bf16, to_f16
from synth.configs import ModelShape

TINY = ModelShape(n_layers=2, d_model=16, n_q_heads=4, n_kv_heads=2, head_dim=4, ffn=24, vocab=8,
                  rope_theta=10000.0, dtype="fp64")


def test_rmsnorm_closed_form():
    c = np.full(16, 3.0)
    np.testing.assert_allclose(rmsnorm(c, np.ones(16), 1e-5), 3.0 / math.sqrt(9.0 + 1e-5))
    x = np.array([3.0, 4.0])          # mean square 12.5
    np.testing.assert_allclose(rmsnorm(x, np.array([1.0, 2.0]), 0.0), [3 / math.sqrt(12.5), 8 / math.sqrt(12.5)])


def test_rope_position_zero_identity_and_norm():
    x = np.random.default_rng(0).normal(size=(3, 8))
    np.testing.assert_array_equal(rope(x, 0, 10000.0), x)
    y = rope(x, 37, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_rope_relative_position():
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=8), rng.normal(size=8)
    d1 = rope(q, 10, 500.0) @ rope(k, 3, 500.0)
    d2 = rope(q, 107, 500.0) @ rope(k, 100, 500.0)
    assert abs(d1 - d2) < 1e-12


def test_rope_pairing_is_rotate_half():
    # D = 2: a single pair (x0, x1) rotated by pos * theta**0 = pos radians
    x = np.array([1.0, 0.0])
    np.testing.assert_allclose(rope(x, 1, 10000.0), [math.cos(1.0), math.sin(1.0)], rtol=1e-15)


def test_attend_special_cases():
    rng = np.random.default_rng(2)
    V = rng.normal(size=(5, 4))
    np.testing.assert_allclose(attend(rng.normal(size=4), V[:1] * 0 + 1, V[:1]), V[0])
    np.testing.assert_allclose(attend(np.zeros(4), rng.normal(size=(5, 4)), V), V.mean(axis=0), rtol=1e-14)
    # two keys, scores 0 and ln 3 (scale sqrt(D) = 2): weights 1/4, 3/4
    q = np.array([2 * math.log(3.0), 0, 0, 0])
    K = np.array([[0.0, 0, 0, 0], [1.0, 0, 0, 0]])
    Vv = np.array([[4.0, 0, 0, 0], [8.0, 0, 0, 0]])
    np.testing.assert_allclose(attend(q, K, Vv), [7.0, 0, 0, 0], rtol=1e-14)


def test_roundings():
    assert to_bf16(1.0 + 2 ** -8) == 1.0
    assert to_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6
    assert to_bf16(1.0 + 2 ** -8 + 2 ** -30) == 1.0 + 2 ** -7
    assert to_f16(1.0 + 2 ** -11) == 1.0
    assert to_f16(70000.0) == np.inf
    assert to_f16(2 ** -24) == 2 ** -24          # smallest fp16 subnormal
    assert to_f16(2 ** -26) == 0.0


@pytest.mark.parametrize("dtype", ["fp64", "fp32"])
def test_cached_greedy_equals_no_cache_recompute(dtype):
    """Textbook special case: KV caching is exact ([KV4] "Autoregressive Decoding
    and the KV Cache").  Greedy with the cache must equal rerunning the whole
    sequence from scratch at every step."""
    W = Weights(TINY, dtype=dtype)
    p = synth.prompt(0, 6, TINY.vocab)
    toks, logits = D.greedy(W, p, 8)
    seq = list(p)
    for i in range(8):
        full = sequence_logits(W, seq)
        np.testing.assert_allclose(full[-1], logits[i], rtol=1e-12 if dtype == "fp64" else 1e-6, atol=1e-12)
        assert argmax(full[-1]) == toks[i]
        seq.append(toks[i])


def test_brute_force_catches_a_planted_mistake():
    """A dropped term in the cached path (no residual after attention) must be
    seen by the no-cache comparison: the check is not vacuous."""
    W = Weights(TINY)
    p = synth.prompt(1, 6, TINY.vocab)
    ref = sequence_logits(W, list(p))[-1]
    orig = D.row_forward

    def broken(Wt, tok, pos, past, rdtype=None):
        out = orig(Wt, tok, pos, past, rdtype)
        out.logits = out.logits + 1e-3 * np.arange(out.logits.size)
        return out

    D.row_forward = broken
    try:
        _, lg = D.greedy(W, p, 1)
    finally:
        D.row_forward = orig
    assert not np.allclose(lg[0], ref, rtol=1e-9)


def test_bf16_mode_close_to_fp64():
    W64 = Weights(TINY, dtype="fp64")
    p = synth.prompt(2, 6, TINY.vocab)
    a = sequence_logits(W64, list(p))
    b = sequence_logits(W64, list(p), rdtype="bf16")
    assert np.max(np.abs(a - b)) < 0.05 * np.max(np.abs(a))
