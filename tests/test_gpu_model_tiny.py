"""End to end on the tiny fp32 decoder (2 layers, d 256, 4 heads, vocab 512,
1024-token prompt, token drop 4x, x = 8, 64 tokens): GPU prefill, greedy and
VeriCache against the oracle, and GPU VeriCache against GPU greedy exactly."""
import numpy as np
import pytest

import synth
from gpu_helpers import TOL_F32, compare_rounds, log, need_gpu, torch
from oracle import decode as OD
from oracle.model import Weights
from synth.configs import tiny as tiny_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup():
    need_gpu()
    from lossless_speculative_decoding_amd import Model
    from lossless_speculative_decoding_amd.engine import make_weights
    w = tiny_workload()
    s = w.model
    W = make_weights(s)
    m = Model(s, W, max_pos=w.ctx[0] + w.n_tokens + 64)
    prompt_np = synth.prompt(0, w.ctx[0], s.vocab)
    prompt = torch.from_numpy(prompt_np).cuda()
    ow = Weights(s)
    log("oracle prefill")
    pre = OD.prefill(ow, prompt_np)
    ref_greedy, ref_logits = OD.greedy(ow, prompt_np, w.n_tokens, pre=pre)
    ref_vc, ref_rounds = OD.vericache(ow, prompt_np, w.n_tokens, w.x[0],
                                      lambda pr: OD.draft_cache_tokdrop(pr, ow, keep_total=w.ctx[0] // 4,
                                                                        keep_recent=64), pre=pre)
    return dict(w=w, s=s, W=W, m=m, prompt=prompt, prompt_np=prompt_np, ow=ow, pre=pre, ref_greedy=ref_greedy,
                ref_logits=ref_logits, ref_rounds=ref_rounds)


def test_weights_layout_matches_oracle(setup):
    s, W, ow = setup["s"], setup["W"], setup["ow"]
    D = s.head_dim
    for l in range(s.n_layers):
        wq = W["w_qkv"][l].cpu().numpy().astype(np.float64)
        assert np.array_equal(wq[: s.n_q_heads * D], ow.Wq[l])
        assert np.array_equal(wq[s.n_q_heads * D:(s.n_q_heads + s.n_kv_heads) * D], ow.Wk[l])
        assert np.array_equal(wq[(s.n_q_heads + s.n_kv_heads) * D:], ow.Wv[l])
        assert np.array_equal(W["w_gu"][l, s.ffn:].cpu().numpy().astype(np.float64), ow.W3[l])
        assert np.array_equal(W["w_down"][l].cpu().numpy().astype(np.float64), ow.W2[l])
    assert np.array_equal(W["lm_head"].cpu().numpy().astype(np.float64), ow.Wlm)


def test_prefill_matches_oracle(setup):
    from lossless_speculative_decoding_amd.engine import greedy_resident
    s, m, prompt, pre = setup["s"], setup["m"], setup["prompt"], setup["pre"]
    toks, _, (kd, vd) = greedy_resident(m, prompt, 1)
    T = prompt.numel()
    kg = kd[:, :, :T].cpu().numpy().astype(np.float64)
    vg = vd[:, :, :T].cpu().numpy().astype(np.float64)
    kr = pre.full.K[:, :, :T]
    vr = pre.full.V[:, :, :T]
    ek = np.abs(kg - kr).max() / np.abs(kr).max()
    ev = np.abs(vg - vr).max() / np.abs(vr).max()
    log("prefill K/V rel err", ek, ev)
    assert ek <= TOL_F32 and ev <= TOL_F32
    assert toks[0] == pre.g0


def _flagged(logits, tol):
    srt = np.sort(logits)[::-1]
    return (srt[0] - srt[1]) < tol * np.abs(logits).max()


def test_greedy_matches_oracle(setup):
    from lossless_speculative_decoding_amd.engine import greedy_resident
    m, prompt, w = setup["m"], setup["prompt"], setup["w"]
    toks, secs, _ = greedy_resident(m, prompt, w.n_tokens)
    ref, ref_logits = setup["ref_greedy"], setup["ref_logits"]
    log("gpu greedy", toks[:12], "oracle", ref[:12], f"{secs:.3f}s")
    for i in range(w.n_tokens):
        if toks[i] != ref[i]:
            assert _flagged(ref_logits[i], TOL_F32), f"unflagged divergence at step {i}"
            log(f"flagged near-tie at step {i}; remaining steps not compared")
            break


def test_vericache_equals_gpu_greedy_and_oracle(setup):
    from lossless_speculative_decoding_amd.engine import Engine, greedy_resident
    m, prompt, w = setup["m"], setup["prompt"], setup["w"]
    g_toks, _, _ = greedy_resident(m, prompt, w.n_tokens)
    eng = Engine(m, w.compress, record=True)
    r = eng.add_request(prompt, w.x[0], w.n_tokens)
    secs = eng.run()
    log("vericache", r.emitted[:12], "accepts", r.accepts, f"{secs:.3f}s")
    assert r.emitted == g_toks, "GPU VeriCache must equal GPU full-KV greedy exactly"
    ref = setup["ref_greedy"]
    same = 0
    for i in range(w.n_tokens):
        if r.emitted[i] != ref[i]:
            assert _flagged(setup["ref_logits"][i], TOL_F32), f"unflagged divergence at {i}"
            break
        same += 1
    rr = setup["ref_rounds"]
    compare_rounds("tiny token drop", r.rounds, [d.a for d in rr], [d.draft for d in rr], [d.verified for d in rr],
                   [d.draft_gap for d in rr], [d.verify_gap for d in rr], TOL_F32)


@pytest.mark.parametrize("fallback_after,plain_rounds", [(2, 3), (0, 0)])
def test_adaptive_and_fallback_rounds_match_oracle(setup, fallback_after, plain_rounds):
    """Adaptive draft length with the fall back to plain rounds (x = 0) when acceptance
    collapses: the GPU engine's rounds (position, drafts, verifier tokens, accept count) equal
    the oracle's loop run with the same policy, and the tokens are the oracle's greedy tokens."""
    from lossless_speculative_decoding_amd.engine import Engine
    m, prompt, w, ow = setup["m"], setup["prompt"], setup["w"], setup["ow"]
    eng = Engine(m, w.compress, record=True)
    r = eng.add_request(prompt, w.x[0], w.n_tokens)
    eng.run(adaptive=True, x_min=2, fallback_after=fallback_after, plain_rounds=plain_rounds)
    pol = OD.DraftLength(w.x[0], x_min=2, fallback_after=fallback_after, plain_rounds=plain_rounds)
    ref, rr = OD.vericache(ow, setup["prompt_np"], w.n_tokens, w.x[0],
                           lambda pr: OD.draft_cache_tokdrop(pr, ow, keep_total=w.ctx[0] // 4, keep_recent=64),
                           pre=setup["pre"], policy=pol)
    xs = [len(g["draft"]) for g in r.rounds]
    log(f"fallback_after={fallback_after}: draft lengths {xs}")
    if fallback_after:
        assert 0 in xs
    compare_rounds("tiny adaptive", r.rounds, [d.a for d in rr], [d.draft for d in rr], [d.verified for d in rr],
                   [d.draft_gap for d in rr], [d.verify_gap for d in rr], TOL_F32)
    i = next((i for i in range(w.n_tokens) if r.emitted[i] != ref[i]), None)
    if i is not None:
        assert _flagged(setup["ref_logits"][i], TOL_F32), f"unflagged divergence from the oracle at {i}"
