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


def compare_rounds(name, gpu_rounds, ref_a, ref_draft, ref_ver, ref_dgap, ref_vgap, tol):
    """GPU rounds (Engine(record=True)) against an oracle run, round by round, up to the first
    draft or verify token that differs, which must be one the oracle flags as a near-tie (its
    relative top-2 gap below tol).  Equal drafts and verifier tokens give equal accept counts;
    with no divergence at all the number of rounds must be equal too.  Returns the rounds
    compared."""
    for k, rd in enumerate(gpu_rounds):
        if k >= len(ref_a):
            break
        assert len(rd["draft"]) == len(ref_draft[k]), f"{name}: round {k}: draft length differs from the oracle's"
        for what, g, r, gap in (("draft", rd["draft"], ref_draft[k], ref_dgap[k]),
                                ("verify row", rd["verified"], ref_ver[k], ref_vgap[k])):
            for i, (a_, b_) in enumerate(zip(g, r)):
                if int(a_) != int(b_):
                    log(f"{name}: round {k} {what} {i} differs (oracle top-2 gap {gap[i]:.2e}); "
                        f"{k} rounds compared before it")
                    assert gap[i] < tol, f"{name}: round {k} {what} {i}: unflagged divergence from the oracle"
                    return k
        assert rd["a"] == int(ref_a[k]), f"{name}: round {k}: same drafts and verifier tokens, other accept count"
    assert len(gpu_rounds) == len(ref_a), f"{name}: same rounds, but {len(gpu_rounds)} against {len(ref_a)}"
    log(f"{name}: all {len(ref_a)} rounds equal the oracle's (accepts {[int(a) for a in ref_a]})")
    return len(ref_a)
