"""The stored oracle run of the small GQA decoder (tests/golden/gqa_model_oracle.npz, written by
tests/golden/make_gqa_model_golden.py from oracle/ alone) is self-consistent: the prompt is
the seeded one, every compressor's VeriCache tokens equal full-KV greedy's ([VC1] "The Core
Idea": identical outputs), and every round follows the accept rule and the position update."""
import os

import numpy as np

import synth
from gqa_model_case import GOLDEN, N, PROMPT_SEED, SHAPE, SPECS, T, X, keep_total
from oracle.decode import accept

G = np.load(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", GOLDEN))


def test_prompt_and_greedy():
    assert np.array_equal(G["prompt"], synth.prompt(PROMPT_SEED, T, SHAPE.vocab))
    assert G["greedy_tokens"].shape == (N,)
    lg = G["greedy_logits_head"]
    assert [int(np.argmax(r)) for r in lg] == G["greedy_tokens"][:4].tolist()


def test_every_compressor_is_lossless_and_rounds_are_consistent():
    for name, spec in SPECS.items():
        toks = G[f"{name}_tokens"].tolist()
        assert toks == G["greedy_tokens"].tolist(), name
        out = [toks[0]]
        pos = T
        for k in range(len(G[f"{name}_a"])):
            d, v, a = G[f"{name}_draft"][k].tolist(), G[f"{name}_verified"][k].tolist(), int(G[f"{name}_a"][k])
            assert len(d) == X and len(v) == X + 1
            assert int(G[f"{name}_pos"][k]) == pos
            a2, emitted = accept(d, v)
            assert a2 == a
            out += emitted
            pos += a + 1
        assert out[:N] == toks and len(out) >= N
        if spec.kind == "tokdrop":
            idx = G[f"{name}_idx"]
            assert idx.shape == (SHAPE.n_layers, SHAPE.n_kv_heads, keep_total(spec))
            assert all(np.all(np.diff(idx[l, j]) > 0) for l in range(SHAPE.n_layers) for j in range(SHAPE.n_kv_heads))
            if spec.keep_recent:
                assert np.array_equal(idx[:, :, -spec.keep_recent:][0, 0], np.arange(T - spec.keep_recent, T))
