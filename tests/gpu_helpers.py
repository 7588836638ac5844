"""Helpers shared by the GPU parity tests (device upload, tolerance checks)."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_speculative_decoding_amd  # noqa: F401  (fails loudly if the library is missing)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> "torch.Tensor":
    """uint16 bf16 bit patterns -> device bfloat16 tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_f32(x: np.ndarray) -> "torch.Tensor":
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_f64(t: "torch.Tensor") -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bytes_of(t: "torch.Tensor") -> bytes:
    return t.detach().cpu().numpy().tobytes()


def row_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Per-row relative L-infinity error max|g - r| / max|r| (rows = last axis), max over rows."""
    g = gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((np.abs(g - r).max(axis=1) / den).max())


TOL_BF16 = 2e-3
TOL_F32 = 1e-5
