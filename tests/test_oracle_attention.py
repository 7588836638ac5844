"""Single-layer workload oracle: verify rows against single-row calls, and the
quantized draft output against a direct dequantize-then-attend."""
import numpy as np

from oracle import attention as A
from oracle.compress import Quantized
from oracle.model import attend


def test_head_inputs_shapes_and_outliers():
    inp = A.head_inputs(1, 2, 256, 8, 32, 128, 4)
    assert inp["K"].shape == (256, 128) and inp["qv"].shape == (4, 4, 128) and inp["qd"].shape == (4, 128)
    col_std = inp["K"].std(axis=0)
    big = np.argsort(col_std)[-4:]
    assert sorted(big.tolist()) == sorted(inp["outl"].tolist())


def test_verify_rows_match_single_row_calls():
    inp = A.head_inputs(0, 0, 128, 8, 32, 128, 3)
    full = A.verify_output(inp)
    for i in range(3):
        K = np.concatenate([inp["K"], inp["tK"][: i + 1]])
        V = np.concatenate([inp["V"], inp["tV"][: i + 1]])
        for g in range(4):
            np.testing.assert_array_equal(full[i, g], attend(inp["qv"][i, g], K, V))


def test_draft_output_uses_dequantized_cache():
    inp = A.head_inputs(0, 1, 256, 8, 32, 128, 1)
    o = A.draft_output(inp, 4, 128)
    q = Quantized(inp["K"][None, None], inp["V"][None, None], 4, 128)
    # dequantized values differ from the originals, but not by more than a step
    assert np.abs(q.Khat[0, 0] - inp["K"]).max() <= q.ks.astype(float).max() * 0.51 + 1e-3
    o_deq = np.stack([attend(qh, np.concatenate([q.Khat[0, 0], inp["tK"][:1]]),
                             np.concatenate([q.Vhat[0, 0], inp["tV"][:1]])) for qh in inp["qd"]])
    np.testing.assert_array_equal(o, o_deq)
    o_full = np.stack([attend(qh, np.concatenate([inp["K"], inp["tK"][:1]]),
                              np.concatenate([inp["V"], inp["tV"][:1]])) for qh in inp["qd"]])
    assert not np.allclose(o, o_full)              # the draft cache is lossy
