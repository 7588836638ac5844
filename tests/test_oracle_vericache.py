"""The pages' central invariant: VeriCache emits exactly the full-KV greedy
tokens ([VC1] "The Core Idea" and "Final Takeaways"; [VC3] "是什么"), for any
draft horizon, any compressor, and even an adversarial drafter."""
import random

import numpy as np
import pytest

import synth
from oracle import decode as D
from oracle.model import Weights
from synth.configs import ModelShape
from synth.configs import tiny as tiny_workload

TINY = ModelShape(n_layers=2, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=48, vocab=16,
                  rope_theta=10000.0, dtype="fp32")


@pytest.fixture(scope="module")
def tiny():
    W = Weights(TINY)
    p = synth.prompt(3, 48, TINY.vocab)
    pre = D.prefill(W, p, obs_window=8)
    ref, _ = D.greedy(W, p, 30, pre=pre)
    return W, p, pre, ref


@pytest.mark.parametrize("x", range(1, 9))
@pytest.mark.parametrize("kind", ["tokdrop", "keynorm", "quant2", "quant4", "identity"])
def test_vericache_equals_greedy(tiny, x, kind):
    W, p, pre, ref = tiny
    mk = {
        "tokdrop": lambda pr: D.draft_cache_tokdrop(pr, W, keep_total=12, keep_recent=4),
        "keynorm": lambda pr: D.draft_cache_keynorm(pr, W, keep_total=10),
        "quant2": lambda pr: D.draft_cache_quant(pr, W, bits=2, group=8),
        "quant4": lambda pr: D.draft_cache_quant(pr, W, bits=4, group=8),
        "identity": D.draft_cache_identity,
    }[kind]
    out, rounds = D.vericache(W, p, 30, x, mk, pre=pre)
    assert out == ref
    for r in rounds:
        assert len(r.emitted) == r.a + 1 and 0 <= r.a <= x
        assert len(r.verified) == x + 1
        if r.a == x:
            assert r.emitted[-1] == r.verified[x]
    if kind == "identity":
        assert all(r.a == x for r in rounds)   # bonus token every round


def test_adversarial_drafter_still_lossless(tiny):
    W, p, pre, ref = tiny
    rng = random.Random(0)
    out, rounds = D.vericache(W, p, 30, 4, D.draft_cache_identity, pre=pre,
                              drafter=lambda r, pend, own: [rng.randrange(TINY.vocab) for _ in own])
    assert out == ref
    assert sum(r.a == 0 for r in rounds) >= len(rounds) // 2


def test_bf16_model_vericache_equals_greedy():
    W = Weights(TINY, dtype="bf16")
    p = synth.prompt(4, 40, TINY.vocab)
    pre = D.prefill(W, p, obs_window=8)
    ref, _ = D.greedy(W, p, 20, pre=pre)
    out, _ = D.vericache(W, p, 20, 5, lambda pr: D.draft_cache_quant(pr, W, bits=3, group=8), pre=pre)
    assert out == ref


@pytest.mark.slow
def test_tiny_workload_full_run():
    w = tiny_workload()
    W = Weights(w.model)
    p = synth.prompt(0, w.ctx[0], w.model.vocab)
    pre = D.prefill(W, p)
    ref, _ = D.greedy(W, p, w.n_tokens, pre=pre)
    out, rounds = D.vericache(W, p, w.n_tokens, w.x[0],
                              lambda pr: D.draft_cache_tokdrop(pr, W, keep_total=256, keep_recent=64), pre=pre)
    assert out == ref and len(out) == 64
    assert 1 + sum(len(r.emitted) for r in rounds) >= 64      # g0 comes from the prefill


def test_draft_length_policy_rules():
    """Growth on a fully kept round, a + 1 after a rejection, the fall back to
    plain rounds after consecutive empty rounds, and the probe afterwards."""
    p = D.DraftLength(8, x_min=2, fallback_after=3, plain_rounds=2)
    seq = []
    for a in [8, 3, 4, 0, 0, 0, 0, 0, 1, 2, 0]:
        seq.append(p.x)
        p.after(a)
    # x: 8 -> (kept all) 8 -> (a=3) 4 -> (kept all) 8 -> 2,2,2 (zeros) -> plain 0,0 -> probe 2 ...
    assert seq == [8, 8, 4, 8, 2, 2, 0, 0, 2, 2, 4]
    q = D.DraftLength(4, fallback_after=0)
    for _ in range(10):
        q.after(0)
    assert q.x == 1                                     # no fall back when it is off


@pytest.mark.parametrize("fallback_after", [0, 1, 2])
def test_adaptive_and_fallback_stay_lossless(tiny, fallback_after):
    W, p, pre, ref = tiny
    pol = D.DraftLength(6, x_min=1, fallback_after=fallback_after, plain_rounds=3)
    out, rounds = D.vericache(W, p, 30, 6, lambda pr: D.draft_cache_tokdrop(pr, W, keep_total=12, keep_recent=4),
                              pre=pre, policy=pol)
    assert out == ref
    xs = [len(r.draft) for r in rounds]
    if fallback_after:
        assert 0 in xs                                  # some rounds decoded plainly
        assert all(len(r.emitted) == 1 for r in rounds if not r.draft)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_matrix_prefill_equals_row_prefill(dtype):
    """The matrix-form prefill stores the same K/V, observation queries, last logits and first
    token as the row-at-a-time prefill (only the float64 summation order differs)."""
    W = Weights(TINY, dtype=dtype)
    p = synth.prompt(4, 40, TINY.vocab)
    a, b = D.prefill(W, p, obs_window=8), D.prefill_matrix(W, p, obs_window=8)
    assert a.full.n == b.full.n == 40 and a.g0 == b.g0
    for x, y in ((a.full.K[:, :, :40], b.full.K[:, :, :40]), (a.full.V[:, :, :40], b.full.V[:, :, :40]),
                 (a.q_obs, b.q_obs)):
        assert np.allclose(x, y, rtol=1e-6, atol=0)
    assert np.allclose(a.last_logits, b.last_logits, rtol=1e-9, atol=1e-12)
