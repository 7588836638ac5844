"""Projection GEMM (vc_linear) against its definition y = x w^T, evaluated in float64.

The GPU sums bf16 (or fp32) products in float32.  Every bf16 x bf16 product is
exact in float32, so whatever the order of the sums, each output is within
(K u / (1 - K u)) sum_k |x_k w_k| of the exact value (u = 2^-24, recursive
summation bound); the test holds every element to that bound, which a dropped
or repeated k slice, a swapped operand chunk or a wrong output index exceeds
by orders of magnitude on these inputs.  Shapes span the 256 x 256 prefill tile
(several tiles, a ragged last row tile, block counts with and without a
multiple of eight), the 128 x 128 tile (N not a multiple of 256) and the
weight-streaming kernel (M <= 64: one to four 16-row tiles, k ranges of one
to 56 chunks of 256, with and without a 128-long last chunk); the Llama-3-8B projection shapes of a
2048-row prefill chunk are checked on sampled rows.
"""
import numpy as np
import pytest

from gpu_helpers import dev_bf16, dev_f32, log, need_gpu, torch

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _operands(M, N, K, seed, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K)) * np.sqrt(2.0 / (N + K))
    if dtype == "bf16":
        import synth
        xb, wb = synth.bf16_bits_from_f32(x.astype(np.float32)), synth.bf16_bits_from_f32(w.astype(np.float32))
        return (dev_bf16(xb), dev_bf16(wb), synth.bf16_bits_to_f32(xb).astype(np.float64),
                synth.bf16_bits_to_f32(wb).astype(np.float64))
    x32, w32 = x.astype(np.float32), w.astype(np.float32)
    return dev_f32(x32), dev_f32(w32), x32.astype(np.float64), w32.astype(np.float64)


def _check(y, x64, w64, rows, label):
    K = x64.shape[1]
    ref = x64[rows] @ w64.T
    bound = (K * U / (1 - K * U)) * (np.abs(x64[rows]) @ np.abs(w64).T) + 1e-30
    got = y[rows].double().cpu().numpy()
    err = np.abs(got - ref)
    worst = float((err / bound).max())
    log(f"{label}: max |err| / bound = {worst:.3g}, max |err| = {err.max():.3g}")
    assert worst <= 1.0, f"{label}: error {worst:.3g} x the float32 summation bound"


@pytest.mark.parametrize("M,N,K,dtype", [
    (300, 768, 128, "bf16"),      # 2 row tiles (ragged) x 3 column tiles: 6 blocks, plain order
    (2085, 1280, 512, "bf16"),    # 9 x 5 = 45 blocks, ragged last row tile
    (512, 2048, 1024, "bf16"),    # 2 x 8 = 16 blocks: XCD-grouped block order
    (65, 256, 4096, "bf16"),      # one ragged row tile, K of the 8B width
    (200, 384, 256, "bf16"),      # N not a multiple of 256: 128 x 128 tiles
    (33, 512, 1024, "bf16"),      # weight-streaming kernel: 3 row tiles, 4 k chunks (main loop once)
    (16, 1024, 384, "bf16"),      # 1 row tile, 1.5 k chunks (a 128-long last chunk, tail only)
    (20, 512, 640, "bf16"),       # 2 row tiles, 2.5 k chunks
    (40, 768, 1152, "bf16"),      # 3 row tiles, 4.5 k chunks (main loop, then a 3-chunk tail)
    (64, 256, 4096, "bf16"),      # 4 row tiles, 16 k chunks
    (1, 4096, 14336, "bf16"),     # one row, 56 k chunks (the 8B down projection's K)
    (100, 96, 80, "f32"),         # fp32 model's kernel
])
def test_linear_matches_definition(M, N, K, dtype):
    need_gpu()
    x, w, x64, w64 = _operands(M, N, K, seed=M * 7 + N * 3 + K, dtype=dtype)
    from lossless_speculative_decoding_amd import vc_linear
    log(f"vc_linear M={M} N={N} K={K} {dtype}")
    y = vc_linear(x, w)
    y2 = vc_linear(x, w)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "two calls differ"
    _check(y, x64, w64, np.arange(M), f"{M}x{N}x{K} {dtype}")


@pytest.mark.parametrize("N,K", [(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)])
def test_linear_llama8b_prefill_shapes_sampled(N, K):
    """One 2048-row prefill chunk at each 8B projection shape (QKV, O, gate/up, down); 48 sampled
    rows (including the first and last of each row tile) against the definition."""
    need_gpu()
    M = 2048
    x, w, x64, w64 = _operands(M, N, K, seed=N + K, dtype="bf16")
    from lossless_speculative_decoding_amd import vc_linear
    log(f"vc_linear M={M} N={N} K={K} bf16 (sampled rows)")
    y = vc_linear(x, w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(N)
    rows = np.unique(np.concatenate([np.arange(0, M, 256), np.arange(255, M, 256), rng.integers(0, M, 32)]))
    _check(y, x64, w64, rows, f"{M}x{N}x{K}")
    assert torch.isfinite(y).all()
