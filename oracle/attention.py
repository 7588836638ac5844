"""Oracle attention for the single-layer GQA workload (decode over a quantized
cache, verification over the full cache).

Plain definition: o_h = sum_t softmax_t(q_h . k_t / sqrt(D)) v_t over the keys
visible to the row, in float64.  The draft row at position T sees the
dequantized cache [0, Tq), the unquantized residual rows [Tq, T) and its own
row; verify row i (position T + i) sees the full cache [0, T) and tail rows
0..i ([VC1] "The Core Idea": the verifier checks all drafted positions in one
pass, each against the full cache and the draft prefix before it).

Pins (tests/test_oracle_attention.py): one key gives o = v; q = 0 gives the
mean of V; a two-key case with a closed-form softmax; and the row-i verify
output equals a single-row call over the same key set.
"""
from __future__ import annotations

import numpy as np

import synth

from .compress import Quantized
from .model import attend


def head_inputs(b: int, j: int, T: int, Hkv: int, Hq: int, D: int, n_rows: int, n_outl: int = 4,
                outl_scale: float = 10.0, seed: int = 0):
    """float64 values of one (request, KV head) slice of the single-layer workload."""
    G = Hq // Hkv
    outl = synth.outlier_channels_for(b, j, Hkv, D, n_outl, seed)
    f = lambda bits: synth.bf16_bits_to_f32(bits).astype(np.float64)
    K = f(synth.att_head(synth.S_ATT_K, b, j, T, Hkv, D, outl, outl_scale, seed))
    V = f(synth.att_head(synth.S_ATT_V, b, j, T, Hkv, D, outl, outl_scale, seed))
    tK = f(synth.att_head(synth.S_ATT_TK, b, j, n_rows, Hkv, D, None, 1.0, seed))
    tV = f(synth.att_head(synth.S_ATT_TV, b, j, n_rows, Hkv, D, None, 1.0, seed))
    qd = f(synth.att_queries(synth.S_ATT_QD, b, 1, Hq, D, seed))[0, j * G:(j + 1) * G]          # [G][D]
    qv = f(synth.att_queries(synth.S_ATT_QV, b, n_rows, Hq, D, seed))[:, j * G:(j + 1) * G]     # [rows][G][D]
    return dict(K=K, V=V, tK=tK, tV=tV, qd=qd, qv=qv, outl=outl)


def draft_output(inp: dict, bits: int, group: int):
    """[G][D] draft-step attention over the quantized cache + residual + own row."""
    q = Quantized(inp["K"][None, None], inp["V"][None, None], bits, group)
    K = np.concatenate([q.rows_K()[0, 0], inp["tK"][:1]])
    V = np.concatenate([q.rows_V()[0, 0], inp["tV"][:1]])
    return np.stack([attend(qh, K, V) for qh in inp["qd"]])


def verify_output(inp: dict, rows=None):
    """[rows][G][D]: verify row i sees the full cache and tail rows 0..i."""
    n = inp["qv"].shape[0]
    rows = range(n) if rows is None else rows
    out = []
    for i in rows:
        K = np.concatenate([inp["K"], inp["tK"][: i + 1]])
        V = np.concatenate([inp["V"], inp["tV"][: i + 1]])
        out.append(np.stack([attend(qh, K, V) for qh in inp["qv"][i]]))
    return np.stack(out)
