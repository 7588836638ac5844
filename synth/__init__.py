"""Seeded synthetic inputs, shared by the CPU oracle and the GPU tests.

This module generates inputs only (weights, prompt ids, K/V/Q tensors and the
per-request draw of context lengths and draft horizons).  It holds none of the
method's arithmetic: no attention, no compression, no decoding.

Generator
---------
A counter-based SplitMix64 (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; Vigna's reference ``splitmix64.c``):

    z(c)  = mix(c + 0x9E3779B97F4A7C15)           (the generator's "next" from state c)
    mix(x): x ^= x >> 30; x *= 0xBF58476D1CE4E5B9; x ^= x >> 27; x *= 0x94D049BB133111EB; x ^= x >> 31
    c     = stream * 2**40 + seed * 2**32 + index  (seed < 256, stream < 2**24, index < 2**32)
    u     = (z >> 40) * 2**-24                     (24-bit uniform in [0, 1))

Derived draws (all arithmetic in float64):
    xavier(fan_in, fan_out): w = (2u - 1) * sqrt(6 / (fan_in + fan_out))
    normal:  element i uses u1 = u(2i), u2 = u(2i + 1);  n = sqrt(-2 ln(1 - u1)) * cos(2 pi u2)
    ids:     (z >> 32) mod V
Storage rounding: float64 -> float32 (round to nearest even); bfloat16 values
are then taken from the float32 by round-to-nearest-even on the top 16 bits.
The GPU library carries its own implementation of the same definition for
inputs too large to generate on the host; tests compare the two bit for bit.
"""
from __future__ import annotations

import math

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


# --------------------------------------------------------------------------
# stream-id table: every tensor / draw has a fixed stream id
# --------------------------------------------------------------------------
S_EMBED = 1
S_LMHEAD = 2
S_PROMPT = 100          # + request index
S_ATT_K = 200           # single-layer attention workload: K, V, draft q, verify q, tail K, tail V, outliers
S_ATT_V = 201
S_ATT_QD = 202
S_ATT_QV = 203
S_ATT_TK = 204
S_ATT_TV = 205
S_ATT_OUTL = 206
S_CTXLEN = 300          # mixed-batch context lengths
S_XDRAW = 301           # mixed-batch draft horizons
S_LOGITS = 400          # synthetic logits rows (sampling tests): + case index
S_LAYER0 = 1000         # + 16 * layer + tensor id
T_WQ, T_WK, T_WV, T_WO, T_W1, T_W3, T_W2 = range(7)


def layer_stream(layer: int, tensor: int) -> int:
    return S_LAYER0 + 16 * layer + tensor


def _counters(stream: int, seed: int, start: int, n: int) -> np.ndarray:
    assert 0 <= seed < 256 and 0 <= stream < (1 << 24)
    assert 0 <= start and start + n <= (1 << 32), "index range exceeds 2**32"
    base = np.uint64((stream << 40) + (seed << 32))
    return base + np.arange(start, start + n, dtype=np.uint64)


def splitmix64(c: np.ndarray) -> np.ndarray:
    """z(c) for a uint64 array of counters (wrapping uint64 arithmetic)."""
    with np.errstate(over="ignore"):
        z = c + np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        return z ^ (z >> np.uint64(31))


_CHUNK = 1 << 22


def _uniform_chunk(stream: int, seed: int, start: int, n: int, out: np.ndarray) -> None:
    z = splitmix64(_counters(stream, seed, start, n))
    out[:] = (z >> np.uint64(40)).astype(np.float64) * (2.0 ** -24)


def uniform(stream: int, n: int, seed: int = 0, start: int = 0) -> np.ndarray:
    """u(start + i), i < n; large draws are evaluated in chunks on a thread pool
    (numpy releases the GIL), which changes nothing in the values."""
    out = np.empty(n, dtype=np.float64)
    if n <= _CHUNK:
        _uniform_chunk(stream, seed, start, n, out)
        return out
    import concurrent.futures as cf
    import os
    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(lambda o: _uniform_chunk(stream, seed, start + o, min(_CHUNK, n - o), out[o:o + _CHUNK]),
                    range(0, n, _CHUNK)))
    return out


def xavier(stream: int, shape, fan_in: int, fan_out: int, seed: int = 0, start: int = 0) -> np.ndarray:
    """Xavier-uniform draw in float64 (not yet rounded to a storage type)."""
    n = int(np.prod(shape))
    a = math.sqrt(6.0 / (fan_in + fan_out))
    return ((2.0 * uniform(stream, n, seed, start) - 1.0) * a).reshape(shape)


def normal(stream: int, shape, seed: int = 0, start: int = 0) -> np.ndarray:
    """Box-Muller standard normals in float64; element i uses counters 2i, 2i+1."""
    n = int(np.prod(shape))
    u = uniform(stream, 2 * n, seed, 2 * start)
    u1, u2 = u[0::2], u[1::2]
    return (np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * math.pi * u2)).reshape(shape)


def ids(stream: int, n: int, vocab: int, seed: int = 0, start: int = 0) -> np.ndarray:
    z = splitmix64(_counters(stream, seed, start, n))
    return ((z >> np.uint64(32)) % np.uint64(vocab)).astype(np.int32)


# --------------------------------------------------------------------------
# storage rounding of generated values
# --------------------------------------------------------------------------
def f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits_from_f32(x32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of float32 values to bfloat16; returns uint16 bit patterns."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gen_bf16(x64: np.ndarray) -> np.ndarray:
    """float64 draw -> bfloat16 bit patterns (via float32, both steps nearest-even)."""
    return bf16_bits_from_f32(f32(x64))


# --------------------------------------------------------------------------
# workload-level draws
# --------------------------------------------------------------------------
def prompt(request: int, length: int, vocab: int, seed: int = 0) -> np.ndarray:
    return ids(S_PROMPT + request, length, vocab, seed)


def mixed_context_lengths(n_req: int, lo: int = 8192, hi: int = 131072, seed: int = 0) -> np.ndarray:
    """Log-uniform context lengths: floor(exp(ln lo + u * ln(hi / lo)))."""
    u = uniform(S_CTXLEN, n_req, seed)
    return np.floor(np.exp(math.log(lo) + u * math.log(hi / lo))).astype(np.int64)


def mixed_draft_horizons(n_req: int, choices=(16, 24, 32, 40), seed: int = 0) -> np.ndarray:
    z = splitmix64(_counters(S_XDRAW, seed, 0, n_req))
    return np.asarray(choices, dtype=np.int64)[((z >> np.uint64(32)) % np.uint64(len(choices))).astype(np.int64)]


def outlier_channels(n_heads_total: int, head_dim: int, n_out: int = 4, seed: int = 0) -> np.ndarray:
    """n_out distinct channel indices per KV head, drawn by a partial Fisher-Yates shuffle.

    Head h uses uniforms u(h * n_out + k), k < n_out: swap position k with
    k + floor(u * (head_dim - k)).  Returns int32 [n_heads_total][n_out].
    """
    out = np.zeros((n_heads_total, n_out), dtype=np.int32)
    u = uniform(S_ATT_OUTL, n_heads_total * n_out, seed)
    for h in range(n_heads_total):
        perm = list(range(head_dim))
        for k in range(n_out):
            j = k + int(u[h * n_out + k] * (head_dim - k))
            perm[k], perm[j] = perm[j], perm[k]
        out[h] = perm[:n_out]
    return out


# --------------------------------------------------------------------------
# single-layer attention workload tensors (Llama-3-8B head shapes)
# --------------------------------------------------------------------------
def att_head(stream: int, b: int, j: int, rows: int, n_heads: int, head_dim: int, outl=None,
             outl_scale: float = 10.0, seed: int = 0) -> np.ndarray:
    """bf16 bit patterns [rows][head_dim] of tensor `stream`, laid out [B][n_heads][rows][D]
    in counter order, for request b, head j.  Columns listed in `outl` are scaled
    by outl_scale before storage rounding."""
    start = ((b * n_heads + j) * rows) * head_dim
    x = normal(stream, (rows, head_dim), seed, start)
    if outl is not None:
        x[:, np.asarray(outl)] *= outl_scale
    return gen_bf16(x)


def att_queries(stream: int, b: int, rows: int, n_q_heads: int, head_dim: int, seed: int = 0) -> np.ndarray:
    """bf16 bits [rows][n_q_heads][D] of a query tensor laid out [B][rows][Hq][D]."""
    start = b * rows * n_q_heads * head_dim
    return gen_bf16(normal(stream, (rows, n_q_heads, head_dim), seed, start))


def outlier_channels_for(b: int, j: int, n_kv_heads: int, head_dim: int, n_out: int = 4, seed: int = 0):
    """Outlier channel indices of request b, KV head j (head number b * Hkv + j)."""
    h = b * n_kv_heads + j
    return outlier_channels(h + 1, head_dim, n_out, seed)[h]
