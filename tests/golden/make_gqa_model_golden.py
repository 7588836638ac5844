"""Writes gqa_model_oracle.npz beside this script: what the oracle computes for the small bf16
GQA decoder of tests/gqa_model_case.py -- full-KV greedy decoding and the VeriCache loop with
each compressor, with the relative top-2 gap of every greedy, draft and verify row, and the
kept sets of the token-drop caches with their top-k boundary margins.

Calls only oracle/ and synth/ (seeded inputs).  Run from the repository root:
    python tests/golden/make_gqa_model_golden.py
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, os.path.dirname(HERE))

import synth  # noqa: E402
from gqa_model_case import GOLDEN, N, PROMPT_SEED, SHAPE, SPECS, T, X, keep_total  # noqa: E402
from oracle import compress as OC  # noqa: E402
from oracle import decode as OD  # noqa: E402
from oracle.model import Weights  # noqa: E402


def boundary_margin(scores: np.ndarray, n_top: int) -> float:
    """Relative gap between the n_top-th and the next candidate score."""
    srt = np.sort(scores)[::-1]
    if n_top >= srt.size:
        return 1.0
    return float((srt[n_top - 1] - srt[n_top]) / max(srt[n_top - 1], 1e-300))


def main():
    t0 = time.time()
    W = Weights(SHAPE)
    p = synth.prompt(PROMPT_SEED, T, SHAPE.vocab)
    pre = OD.prefill(W, p)
    print(f"prefill {time.time() - t0:.0f}s", flush=True)
    out = {"prompt": p.astype(np.int32)}
    toks, logits = OD.greedy(W, p, N, pre=pre)
    out["greedy_tokens"] = np.array(toks, np.int32)
    out["greedy_gap"] = np.array([OD.rel_gap(lg) for lg in logits])
    out["greedy_logits_head"] = np.stack(logits[:4])
    print(f"greedy {time.time() - t0:.0f}s", flush=True)
    L, H = SHAPE.n_layers, SHAPE.n_kv_heads
    for name, spec in SPECS.items():
        if spec.kind == "quant":
            mk = lambda pr, spec=spec: OD.draft_cache_quant(pr, W, bits=spec.bits, group=spec.group)
        elif spec.score == "keynorm":
            kt = keep_total(spec)
            n = pre.full.n
            idx, _, _, sc = OC.tokdrop_keynorm(pre.full.K[:, :, :n], pre.full.V[:, :, :n], kt)
            out[f"{name}_idx"] = np.asarray(idx, np.int32)
            out[f"{name}_margin"] = np.array([[boundary_margin(np.asarray(sc)[l], kt)] * H for l in range(L)])
            mk = lambda pr, kt=kt: OD.draft_cache_keynorm(pr, W, keep_total=kt)
        else:
            kt = keep_total(spec)
            n = pre.full.n
            idx, _, _, sc = OC.tokdrop(pre.full.K[:, :, :n], pre.full.V[:, :, :n], pre.q_obs, kt, spec.keep_recent,
                                       SHAPE.group)
            out[f"{name}_idx"] = np.asarray(idx, np.int32)
            out[f"{name}_margin"] = np.array([[boundary_margin(np.asarray(sc)[l, j], kt - spec.keep_recent)
                                               for j in range(H)] for l in range(L)])
            mk = lambda pr, kt=kt, spec=spec: OD.draft_cache_tokdrop(pr, W, keep_total=kt,
                                                                      keep_recent=spec.keep_recent)
        vt, rounds = OD.vericache(W, p, N, X, mk, pre=pre)
        assert vt == toks, f"{name}: oracle VeriCache differs from oracle greedy"
        out[f"{name}_tokens"] = np.array(vt, np.int32)
        out[f"{name}_pos"] = np.array([r.pos for r in rounds], np.int32)
        out[f"{name}_a"] = np.array([r.a for r in rounds], np.int32)
        out[f"{name}_draft"] = np.array([r.draft for r in rounds], np.int32)
        out[f"{name}_verified"] = np.array([r.verified for r in rounds], np.int32)
        out[f"{name}_draft_gap"] = np.array([r.draft_gap for r in rounds])
        out[f"{name}_verify_gap"] = np.array([r.verify_gap for r in rounds])
        print(f"{name}: accepts {[r.a for r in rounds]} ({time.time() - t0:.0f}s)", flush=True)
    np.savez_compressed(os.path.join(HERE, GOLDEN), **out)


if __name__ == "__main__":
    main()
