"""Storage roundings used by the oracle (float64 in, float64 out).

Each function returns the float64 value of the nearest representable number
of the storage type, ties to even, computed directly from the float64 input
(no intermediate float32 step).
"""
from __future__ import annotations

import numpy as np


def _round_sig(x: np.ndarray, sig_bits: int, min_exp: int) -> np.ndarray:
    """Round to `sig_bits` significant bits; values below 2**(min_exp-1) use the
    subnormal quantum 2**(min_exp - sig_bits)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, min_exp)
    q = np.ldexp(1.0, e - sig_bits)
    return np.rint(x / q) * q               # np.rint: round half to even


def to_bf16(x):
    """bfloat16: 8 significant bits, smallest normal 2**-126 (frexp exponent -125)."""
    return _round_sig(x, 8, -125)


def to_f16(x):
    """IEEE half: 11 significant bits, smallest normal 2**-14, overflow to inf."""
    r = _round_sig(x, 11, -13)
    return np.where(np.abs(r) > 65504.0, np.copysign(np.inf, r), r)


def to_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def identity(x):
    return np.asarray(x, dtype=np.float64)


def storage_round(dtype: str):
    return {"bf16": to_bf16, "fp32": to_f32, "fp64": identity}[dtype]
