"""Model pins: closed forms for RMSNorm and RoPE, and the cached greedy decode
against a brute-force no-cache recomputation."""
import math

import numpy as np
import pytest

import synth
from oracle import decode as D
from oracle.model import Weights, argmax, attend, rmsnorm, rope, row_forward, sequence_logits, silu
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


def test_rope_frequencies_and_pairing_at_d8():
    """Rotate-half pairing and the frequency exponent at D = 8: unit vector e_i (i < D/2) turns
    towards e_{i + D/2} by the angle pos * theta**(-2i/D); e_{i + D/2} turns towards -e_i."""
    D, theta, pos = 8, 10000.0, 3
    for i in range(D // 2):
        ang = pos * theta ** (-2.0 * i / D)
        e = np.zeros(D)
        e[i] = 1.0
        want = np.zeros(D)
        want[i], want[i + D // 2] = math.cos(ang), math.sin(ang)
        np.testing.assert_allclose(rope(e, pos, theta), want, rtol=1e-14, atol=1e-15)
        e = np.zeros(D)
        e[i + D // 2] = 1.0
        want = np.zeros(D)
        want[i], want[i + D // 2] = -math.sin(ang), math.cos(ang)
        np.testing.assert_allclose(rope(e, pos, theta), want, rtol=1e-14, atol=1e-15)
    # the angles themselves: pos 1 gives 1, theta**-0.25, theta**-0.5, theta**-0.75 radians
    e = np.zeros(D)
    e[1] = 1.0
    np.testing.assert_allclose(rope(e, 1, theta)[[1, 5]], [math.cos(0.1), math.sin(0.1)], rtol=1e-14)


def test_rope_is_complex_multiplication():
    """Rotate-half RoPE equals multiplying z_i = x_i + i x_{i+D/2} by exp(i pos theta_i)."""
    rng = np.random.default_rng(4)
    D, theta, pos = 16, 500000.0, 12345
    x = rng.normal(size=D)
    z = (x[: D // 2] + 1j * x[D // 2:]) * np.exp(1j * pos * theta ** (-np.arange(D // 2) * 2.0 / D))
    np.testing.assert_allclose(rope(x, pos, theta), np.concatenate([z.real, z.imag]), rtol=1e-12, atol=1e-12)


def test_silu_closed_forms():
    """silu(x) = x sigma(x): sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4, silu(0) = 0, and
    silu(x) - silu(-x) = x for every x."""
    l3 = math.log(3.0)
    np.testing.assert_allclose(silu(np.array([l3, -l3, 0.0])), [0.75 * l3, -0.25 * l3, 0.0], rtol=1e-15, atol=0)
    x = np.linspace(-6, 6, 25)
    np.testing.assert_allclose(silu(x) - silu(-x), x, rtol=1e-14, atol=1e-14)
    assert abs(silu(np.array([40.0]))[0] - 40.0) < 1e-15 * 40 * 1e3


def _crafted_ffn_model():
    """One layer, d = 4, one head of 4, ffn 2, vocab 4, eps 0: attention weights zero (the
    attention output is then exactly zero), the embedding row of token 0 is [1, 1, 1, 1],
    the gate projection W1 reads 2 * x0 into unit 0, the up projection W3 reads 3 * x0 into
    unit 0, W2 writes unit 0 back to channel 0, and the LM head is the identity."""
    s = ModelShape(n_layers=1, d_model=4, n_q_heads=1, n_kv_heads=1, head_dim=4, ffn=2, vocab=4,
                   rope_theta=10000.0, dtype="fp64", eps=0.0)
    W = Weights.__new__(Weights)
    W.shape, W.dtype = s, "fp64"
    W.E = np.ones((4, 4))
    W.Wlm = np.eye(4)
    z4 = np.zeros((4, 4))
    W.Wq, W.Wk, W.Wv, W.Wo = [z4], [z4], [z4], [z4]
    W.W1 = [np.array([[2.0, 0, 0, 0], [0, 0, 0, 0]])]
    W.W3 = [np.array([[3.0, 0, 0, 0], [0, 0, 0, 0]])]
    W.W2 = [np.array([[1.0, 0], [0, 0], [0, 0], [0, 0]])]
    W.g1, W.g2, W.gF = [np.ones(4)], [np.ones(4)], np.ones(4)
    return W


def test_swiglu_gate_and_up_assignment():
    """SwiGLU is silu(W1 f) * (W3 f): with gate 2 and up 3 the residual gains 3 * silu(2) =
    6 sigma(2) on channel 0 (with the roles swapped it would gain 2 * silu(3) = 6 sigma(3))."""
    W = _crafted_ffn_model()
    h0 = 1.0 + 6.0 / (1.0 + math.exp(-2.0))
    h = np.array([h0, 1.0, 1.0, 1.0])
    want = h / math.sqrt(np.mean(h * h))
    none = lambda l, j: (np.zeros((0, 4)), np.zeros((0, 4)))
    got = row_forward(W, 0, 5, none).logits
    np.testing.assert_allclose(got, want, rtol=1e-14)
    np.testing.assert_allclose(sequence_logits(W, [0])[-1], want, rtol=1e-14)
    hs = np.array([1.0 + 6.0 / (1.0 + math.exp(-3.0)), 1.0, 1.0, 1.0])
    assert np.max(np.abs(got - hs / math.sqrt(np.mean(hs * hs)))) > 1e-3


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


# ---------------------------------------------------------------- the full-size forms
GQA = ModelShape(n_layers=2, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=48, vocab=37,
                 rope_theta=10000.0, dtype="bf16")


def test_layer_weights_and_embedding_rows_are_the_weights_recipe():
    """LayerWeights (row chunks, on a thread pool or not) and embed_rows give exactly the values
    of Weights."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle.model import LayerWeights, _stored_chunked, embed_rows
    W = Weights(GQA)
    with ThreadPoolExecutor(3) as pool:
        for l in range(GQA.n_layers):
            Lw = LayerWeights(GQA, l, pool=pool)
            for name in ("Wq", "Wk", "Wv", "Wo", "W1", "W3", "W2"):
                assert np.array_equal(getattr(Lw, name)[l], getattr(W, name)[l]), name
        st = synth.layer_stream(1, synth.T_W1)
        assert np.array_equal(_stored_chunked(st, GQA.ffn, GQA.d_model, 0, "bf16", pool, rows=5), W.W1[1])
    toks = [0, 5, 36, 5]
    assert np.array_equal(embed_rows(GQA, toks), W.E[toks])


def test_head_logits_equals_head_forward():
    from concurrent.futures import ThreadPoolExecutor
    from oracle.model import head_forward, head_logits
    W = Weights(GQA)
    rng = np.random.default_rng(3)
    H = to_bf16(rng.standard_normal((3, GQA.d_model)))
    ref = np.stack([head_forward(W, h) for h in H])
    with ThreadPoolExecutor(2) as pool:
        got = head_logits(GQA, H, pool=pool, rows=7)          # 37 rows in chunks of 7
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


@pytest.mark.parametrize("rdtype", ["fp64", "bf16"])
def test_layer_forward_rows_equals_row_by_row(rdtype):
    """n rows through one layer at once against layer_forward one row at a time, each row seeing
    the same cached prefix and the earlier rows of the call (fp64: to rounding of sums; bf16: the
    stored values may differ where a float64 sum sits on a bf16 rounding boundary, by one ulp)."""
    from oracle.model import layer_forward, layer_forward_rows
    W = Weights(GQA)
    rng = np.random.default_rng(7)
    T, n, pos0 = 9, 4, 9
    R = (lambda x: x) if rdtype == "fp64" else to_bf16
    Kp = R(rng.standard_normal((GQA.n_kv_heads, T, GQA.head_dim)))
    Vp = R(rng.standard_normal((GQA.n_kv_heads, T, GQA.head_dim)))
    H = R(rng.standard_normal((n, GQA.d_model)))
    for l in range(GQA.n_layers):
        Hg, Kg, Vg = layer_forward_rows(W, l, H, pos0, Kp, Vp, rdtype)
        ks, vs = [], []
        for i in range(n):
            def past(j, i=i):
                return (np.concatenate([Kp[j]] + [k[j][None] for k in ks]),
                        np.concatenate([Vp[j]] + [v[j][None] for v in vs]))
            h, k, v, _, _ = layer_forward(W, l, H[i], pos0 + i, past, rdtype)
            ks.append(k)
            vs.append(v)
            tol = 1e-12 if rdtype == "fp64" else 2.0 ** -7
            for got, ref in ((Hg[i], h), (Kg[i], k), (Vg[i], v)):
                assert np.abs(got - ref).max() <= tol * np.abs(ref).max(), (l, i)
        H = Hg


def test_layer_forward_rows_catches_a_planted_mistake():
    """A row that also sees the row after it (a causal-mask mistake) changes the outputs."""
    from oracle.model import layer_forward_rows
    W = Weights(GQA)
    rng = np.random.default_rng(8)
    Kp = rng.standard_normal((GQA.n_kv_heads, 5, GQA.head_dim))
    Vp = rng.standard_normal((GQA.n_kv_heads, 5, GQA.head_dim))
    H = rng.standard_normal((3, GQA.d_model))
    ref, _, _ = layer_forward_rows(W, 0, H, 5, Kp, Vp, "fp64")
    # rows 0 and 1 alone: row 0 must not change when row 1 is dropped (it never sees it)
    one, _, _ = layer_forward_rows(W, 0, H[:1], 5, Kp, Vp, "fp64")
    assert np.abs(one[0] - ref[0]).max() <= 1e-12 * np.abs(ref[0]).max()
    # but a prefix with one more key changes every row
    more, _, _ = layer_forward_rows(W, 0, H, 5, np.concatenate([Kp, Kp[:, :1]], 1), np.concatenate([Vp, Vp[:, :1]], 1), "fp64")
    assert np.abs(more - ref).max() > 1e-6
