"""Pins of the oracle's sampled decoding ([VC2] "VeriCache Guide: Lossless
Inference with Lossy KV Caches", "Mathematical Guarantee of Lossless
Correctness"): the generator against numpy's own Philox and the published
known answer, inverse-CDF sampling by exact counting, the rejection rule by
the exact marginal identity and by chi-square tests of emitted frequencies
(with a planted mistake that the test must catch), and temperature 0 against
the greedy loops."""
from fractions import Fraction
import random

import numpy as np
import pytest
from scipy.stats import chisquare

import synth
from oracle import decode as D
from oracle import sampling as S
from oracle.model import Weights, row_forward
from synth.configs import ModelShape

TINY = ModelShape(n_layers=2, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=48, vocab=16,
                  rope_theta=10000.0, dtype="fp32")


# ------------------------------------------------------------------ generator
def test_philox_matches_numpy_philox():
    """numpy.random.Philox is Philox4x64-10; it advances its 256-bit counter
    before each block, so a generator started at counter c first returns the
    block of c + 1."""
    for ctr, key in [([0, 0, 0, 0], [0, 0]), ([5, 7, 9, 11], [123, 456]),
                     ([2 ** 64 - 2, 3, 0, 0], [2 ** 63 + 17, 99]), ([1000, 2, 12345, 0], [0xDEADBEEF, 0])]:
        got = np.random.Philox(counter=np.array(ctr, np.uint64), key=np.array(key, np.uint64)).random_raw(4)
        nxt = list(ctr)
        nxt[0] = (nxt[0] + 1) % 2 ** 64
        if nxt[0] == 0:
            nxt[1] += 1
        assert [int(v) for v in got] == list(S.philox4x64_10(nxt, key)), (ctr, key)


def test_philox_known_answer_all_zero():
    # the all-zero counter and key vector of the generator's published known answers
    assert S.philox4x64_10([0, 0, 0, 0], [0, 0]) == (0x16554D9ECA36314C, 0xDB20FE9D672D0FDC,
                                                      0xD7E772CEE186176B, 0x7E68B68AEC7BA23B)


def test_uniform_grid_and_spread():
    us = [S.uniform(7, s, p, k) for s in range(4) for p in range(40) for k in range(3)]
    for u in us:
        assert 0.0 <= u < 1.0 and u * 2 ** 24 == int(u * 2 ** 24)
    assert len(set(us)) == len(us)
    h = np.histogram(us, bins=8, range=(0, 1))[0]
    assert chisquare(h).pvalue > 1e-3


# ------------------------------------------------------------------ inverse CDF
def test_sample_index_counts_exactly_on_a_grid():
    """With integer weights summing to 16 and u over the 16 grid points, index
    i is chosen exactly w_i times; a zero weight never; u * S on an interval
    edge takes the next index (the running sum must exceed it)."""
    w = [3, 0, 5, 1, 0, 7]
    counts = np.zeros(len(w), int)
    for j in range(16):
        counts[S.sample_index(w, j / 16)[0]] += 1
    assert list(counts) == w
    assert S.sample_index(w, 3 / 16)[0] == 2          # target 3 = C_0 exactly -> next positive weight
    assert S.sample_index([0, 0, 2], 0.0)[0] == 2
    k, m = S.sample_index([1, 1], 0.25)
    assert k == 0 and m == pytest.approx(0.25)


def test_tempered_probs_special_cases():
    z = np.array([1.0, 3.0, 3.0, -np.inf, 0.5])
    p0 = S.tempered_probs(z, 0.0)
    assert list(p0) == [0, 1, 0, 0, 0]                 # temperature 0: lowest index of the maximum
    p1 = S.tempered_probs(z, 1.0)
    assert p1[3] == 0.0 and p1[1] == p1[2] and p1.sum() == pytest.approx(1.0)
    assert p1[0] / p1[4] == pytest.approx(np.exp(0.5))
    p2 = S.tempered_probs(z, 2.0)
    assert p2[1] / p2[0] == pytest.approx(np.exp(1.0))
    for bad in ([1.0, np.nan], [np.inf, 0.0], [-np.inf, -np.inf]):
        assert S.tempered_probs(np.array(bad), 1.0) is None
        assert S.sample_row(np.array(bad), 1.0, 0, 0, 0, S.TARGET)[0] == -1


# ------------------------------------------------------------------ rejection rule
def _rand_dist(rng, n, zeros=0):
    w = [Fraction(rng.randint(1, 30)) for _ in range(n)]
    for i in rng.sample(range(n), zeros):
        w[i] = Fraction(0)
    s = sum(w)
    return [v / s for v in w]


def test_marginal_equals_target_exactly():
    """P(x) = p_d(x) alpha(x) + (1 - sum_y p_d(y) alpha(y)) p_res(x) equals
    p_target(x) exactly, for random rational distributions, with zeros on
    either side and with p_d = p_t."""
    rng = random.Random(5)
    cases = [(_rand_dist(rng, 6), _rand_dist(rng, 6)) for _ in range(20)]
    cases += [(_rand_dist(rng, 7, zeros=3), _rand_dist(rng, 7, zeros=2)) for _ in range(20)]
    p = _rand_dist(rng, 5)
    cases.append((p, list(p)))
    for pt, pd in cases:
        alpha = [S.accept_probability(pt, pd, x) if pd[x] > 0 else Fraction(0) for x in range(len(pt))]
        kept = sum(pd[x] * alpha[x] for x in range(len(pt)))
        res = S.residual(pt, pd)
        if res is None:
            assert kept == 1
            res = [Fraction(0)] * len(pt)
        marg = [pd[x] * alpha[x] + (1 - kept) * res[x] for x in range(len(pt))]
        assert marg == pt


def test_residual_never_returns_a_rejected_candidate():
    rng = np.random.default_rng(3)
    for _ in range(200):
        pt, pd = rng.dirichlet(np.ones(9)), rng.dirichlet(np.ones(9))
        d = int(rng.integers(9))
        u = float(rng.random())
        a, k, _ = S.speculative_accept([pt, pt], [pd], [d], [u], [0.3, 0.7])
        if a == 0:
            assert k != d and pt[d] <= u * pd[d]


PT = np.array([0.05, 0.30, 0.02, 0.18, 0.25, 0.0, 0.12, 0.08])
PD = np.array([0.20, 0.05, 0.10, 0.18, 0.02, 0.15, 0.20, 0.10])


def _one_position_freqs(n, seed):
    counts = np.zeros(len(PT), int)
    rejected = 0
    for t in range(n):
        d, _ = S.sample_index(PD, S.uniform(seed, t, 1, S.DRAFT))
        a, k, _ = S.speculative_accept([PT, PT], [PD], [d], [S.uniform(seed, t, 1, S.ACCEPT)],
                                       [S.uniform(seed, t, 1, S.TARGET), S.uniform(seed, t, 2, S.TARGET)])
        counts[d if a == 1 else k] += 1
        rejected += a == 0
    return counts, rejected / n


def test_chi_square_one_position():
    counts, rej = _one_position_freqs(20000, 11)
    assert 0.3 < rej < 0.7                            # the two distributions differ a lot
    m = PT > 0
    assert counts[~m].sum() == 0                       # a zero-probability target token is never emitted
    assert chisquare(counts[m], PT[m] * counts.sum()).pvalue > 1e-3


def test_chi_square_catches_a_planted_residual_mistake(monkeypatch):
    """Resampling from p_target instead of the residual (a plausible slip)
    makes the emitted distribution wrong; the chi-square test must see it."""
    monkeypatch.setattr(S, "residual_weights", lambda pt, pd: np.asarray(pt, dtype=np.float64))
    counts, _ = _one_position_freqs(20000, 11)
    m = PT > 0
    assert chisquare(counts[m], PT[m] * counts.sum()).pvalue < 1e-6


def test_chi_square_three_drafts_markov_chain():
    """A context-dependent pair of distributions (a Markov chain over 5
    tokens: row s of each matrix is the next-token distribution after s): the
    first three tokens emitted by rounds of x = 3 drafts follow the target
    chain's joint law."""
    rng = np.random.default_rng(8)
    V, x, n = 5, 3, 12000
    Pt = rng.dirichlet(np.ones(V) * 0.8, size=V)
    Pd = rng.dirichlet(np.ones(V) * 0.8, size=V)
    seed, start = 21, 2
    counts = np.zeros((V, V, V), int)
    acc = []
    for t in range(n):
        out, pending, pos = [], start, 10
        while len(out) < 3:
            draft, prev = [], pending
            for i in range(x):
                prev, _ = S.sample_index(Pd[prev], S.uniform(seed, t, pos + 1 + i, S.DRAFT))
                draft.append(prev)
            rows = [pending] + draft
            a, k, _ = S.speculative_accept([Pt[r] for r in rows], [Pd[r] for r in rows[:x]], draft,
                                           [S.uniform(seed, t, pos + 1 + i, S.ACCEPT) for i in range(x)],
                                           [S.uniform(seed, t, pos + 1 + i, S.TARGET) for i in range(x + 1)])
            acc.append(a)
            out += draft[:a] + [k]
            pending, pos = k, pos + a + 1
        counts[out[0], out[1], out[2]] += 1
    exact = Pt[start][:, None, None] * Pt[:, :, None] * Pt[None, :, :]
    assert 0.5 < np.mean(acc) < 2.5
    e = exact.ravel() * n
    keep = e >= 5
    obs = np.append(counts.ravel()[keep], counts.ravel()[~keep].sum())
    exp_ = np.append(e[keep], e[~keep].sum())
    assert chisquare(obs, exp_).pvalue > 1e-3


# ------------------------------------------------------------------ on a model
@pytest.fixture(scope="module")
def tiny():
    W = Weights(TINY)
    p = synth.prompt(3, 48, TINY.vocab)
    pre = D.prefill(W, p, obs_window=8)
    return W, p, pre


def _tokdrop(W):
    return lambda pr: D.draft_cache_tokdrop(pr, W, keep_total=12, keep_recent=4)


def test_temperature_zero_is_greedy(tiny):
    W, p, pre = tiny
    ref, _ = D.greedy(W, p, 30, pre=pre)
    toks, _ = S.sampled_decode(W, p, 30, 0.0, seed=1, pre=pre)
    assert toks == ref
    for x in (1, 4, 7):
        out, rounds = S.vericache_sampled(W, p, 30, x, _tokdrop(W), 0.0, seed=1, pre=pre)
        g_out, g_rounds = D.vericache(W, p, 30, x, _tokdrop(W), pre=pre)
        assert out == ref == g_out
        assert [r.a for r in rounds] == [r.a for r in g_rounds]


def test_temperature_to_zero_limit(tiny):
    """A vanishing temperature draws the greedy token wherever the top two
    logits are apart (the softmax weights of the rest underflow)."""
    W, p, pre = tiny
    ref, _ = D.greedy(W, p, 24, pre=pre)
    toks, _ = S.sampled_decode(W, p, 24, 1e-9, seed=3, pre=pre)
    assert toks == ref
    out, _ = S.vericache_sampled(W, p, 24, 4, _tokdrop(W), 1e-9, seed=3, pre=pre)
    assert out == ref


def test_model_first_tokens_follow_full_kv_law(tiny):
    """On the model: g0 and the next token of sampled VeriCache (token drop,
    x = 3, temperature 1) over many streams follow the full-KV law
    p(g0) p(t1 | g0), computed exactly from the model's rows."""
    W, p, pre = tiny
    tau, n, V = 1.0, 1500, TINY.vocab
    p0 = S.tempered_probs(pre.last_logits, tau)
    T = len(p)
    p1 = np.zeros((V, V))
    for g in range(V):
        full = pre.full.copy()
        o = row_forward(W, g, T, full.rows)
        p1[g] = S.tempered_probs(o.logits, tau)
    counts = np.zeros((V, V), int)
    rej = 0
    for stream in range(n):
        out, rounds = S.vericache_sampled(W, p, 2, 3, _tokdrop(W), tau, seed=4, stream=stream, pre=pre)
        counts[out[0], out[1]] += 1
        rej += rounds[0].a < 3
    assert rej > 0.05 * n                              # the compressed cache's drafts do get rejected
    e = (p0[:, None] * p1).ravel() * n
    keep = e >= 5
    obs = np.append(counts.ravel()[keep], counts.ravel()[~keep].sum())
    exp_ = np.append(e[keep], e[~keep].sum())
    assert chisquare(obs, exp_).pvalue > 1e-3


def test_identity_draft_cache_keeps_every_draft(tiny):
    """With an uncompressed draft cache the two distributions are equal, so
    u * p_d < p_t holds for every u < 1: each round keeps all x drafts and
    draws the bonus token."""
    W, p, pre = tiny
    _, rounds = S.vericache_sampled(W, p, 20, 3, D.draft_cache_identity, 0.8, seed=9, pre=pre)
    assert all(r.a == 3 for r in rounds)
