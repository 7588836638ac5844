"""Oracle decoder: a pre-norm Llama-style model evaluated one row at a time.

The pages never spell out the architecture; the workloads name RMSNorm, RoPE,
SwiGLU and MHA/GQA with Xavier-initialised weights, which is read here as the
usual pre-norm decoder:

    h = E[tok]
    per layer l:
        a = rmsnorm(h) * g1[l]
        q, k, v = Wq a, Wk a, Wv a ; q, k = rope(q, pos), rope(k, pos)   (K is cached after RoPE)
        o_h = sum_t softmax_t(q_h . k_{j(h),t} / sqrt(D)) v_{j(h),t}      over cached rows + own row
        h = h + Wo concat(o)
        f = rmsnorm(h) * g2[l]
        h = h + W2 (silu(W1 f) * (W3 f))
    logits = Wlm (rmsnorm(h) * gF)

Everything is float64.  Between steps the value is rounded to the storage type
(bf16 or fp32) at the points where the GPU path stores a tensor in memory:
norm outputs, q/k/v after RoPE, attention output, the residual after each add,
the SwiGLU product, and the final norm.  Logits stay float64.

Every row goes through ``row_forward`` with the keys visible to it given in
absolute-position order, so a verification row and the greedy row at the same
position are the same computation.  That is the property [KV4] "Autoregressive
Decoding and the KV Cache" states: past rows' K/V do not depend on later
tokens, so caching them is exact.

Pins: tests/test_oracle_model.py checks RMSNorm against its closed form; RoPE
at position 0 (identity), norm preservation, relative-position dependence, the
rotate-half pairing and the frequencies theta**(-2i/D) on unit vectors at D = 8,
and the equivalence with complex multiplication by exp(i pos theta_i); silu at
closed-form points (sigma(ln 3) = 3/4) and its odd-part identity; the SwiGLU
gate/up assignment on a crafted one-layer model; and the cached row-by-row
greedy decode against a brute-force recomputation of the whole sequence in
matrix form with no cache (``sequence_logits``); and the full-size forms at the
end of this file (``LayerWeights``, ``embed_rows``, ``head_logits``,
``layer_forward_rows``) against ``Weights``, ``head_forward`` and
``layer_forward`` on small shapes.
"""
from __future__ import annotations

import math

import numpy as np

import synth
from synth.configs import ModelShape

from .rounding import storage_round


def _stored(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Generated float64 draw -> the value the model stores (input recipe)."""
    if dtype == "bf16":
        return synth.bf16_bits_to_f32(synth.gen_bf16(x64)).astype(np.float64)
    if dtype == "fp32":
        return synth.f32(x64).astype(np.float64)
    return np.asarray(x64, dtype=np.float64)


class Weights:
    """All weights of a model shape, as float64 arrays of the stored values.

    Matrices are [out][in].  Norm gains are ones.  Xavier-uniform for every
    matrix, with fan_in = in, fan_out = out (E is [V][d], Wlm is [V][d]).
    """

    def __init__(self, shape: ModelShape, seed: int = 0, dtype: str | None = None):
        s = shape
        dt = dtype or s.dtype
        self.shape, self.dtype = s, dt
        D = s.head_dim

        def mat(stream, out_dim, in_dim):
            return _stored(synth.xavier(stream, (out_dim, in_dim), in_dim, out_dim, seed), dt)

        self.E = mat(synth.S_EMBED, s.vocab, s.d_model)
        self.Wlm = mat(synth.S_LMHEAD, s.vocab, s.d_model)
        self.Wq, self.Wk, self.Wv, self.Wo, self.W1, self.W3, self.W2 = ([] for _ in range(7))
        for l in range(s.n_layers):
            st = lambda t: synth.layer_stream(l, t)
            self.Wq.append(mat(st(synth.T_WQ), s.n_q_heads * D, s.d_model))
            self.Wk.append(mat(st(synth.T_WK), s.n_kv_heads * D, s.d_model))
            self.Wv.append(mat(st(synth.T_WV), s.n_kv_heads * D, s.d_model))
            self.Wo.append(mat(st(synth.T_WO), s.d_model, s.n_q_heads * D))
            self.W1.append(mat(st(synth.T_W1), s.ffn, s.d_model))
            self.W3.append(mat(st(synth.T_W3), s.ffn, s.d_model))
            self.W2.append(mat(st(synth.T_W2), s.d_model, s.ffn))
        self.g1 = [np.ones(s.d_model) for _ in range(s.n_layers)]
        self.g2 = [np.ones(s.d_model) for _ in range(s.n_layers)]
        self.gF = np.ones(s.d_model)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g, over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope_angles(pos: int, head_dim: int, theta: float) -> np.ndarray:
    """theta_i = pos * theta**(-2i/D), i < D/2."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return pos * theta ** (-2.0 * i / head_dim)


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate-half RoPE on [..., D]: pair (i, i + D/2) is rotated by angle theta_i."""
    D = x.shape[-1]
    ang = rope_angles(pos, D, theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """softmax(K q / sqrt(D)) V for one query row q [D] over keys K, V [n][D]."""
    s = K @ q / math.sqrt(q.shape[-1])
    p = np.exp(s - s.max())
    return (p / p.sum()) @ V


class RowOut:
    __slots__ = ("logits", "k", "v", "q")

    def __init__(self, logits, k, v, q):
        self.logits, self.k, self.v, self.q = logits, k, v, q


def layer_forward(W: Weights, l: int, h: np.ndarray, pos: int, past, rdtype: str | None = None):
    """Layer l on one row: residual stream h [d] (as stored) at position pos.

    past(j) -> (K [n][D], V [n][D]): the rows of layer l, KV head j visible to this
    row, in absolute-position order (this row's own K/V is appended after them).
    Returns (h_out [d], k [Hkv][D], v [Hkv][D], q [Hq][D], o [Hq][D]), each as stored."""
    s = W.shape
    R = storage_round(rdtype or W.dtype)
    D, G, Hq, Hkv = s.head_dim, s.group, s.n_q_heads, s.n_kv_heads
    a = R(rmsnorm(h, W.g1[l], s.eps))
    q = R(rope((W.Wq[l] @ a).reshape(Hq, D), pos, s.rope_theta))
    k = R(rope((W.Wk[l] @ a).reshape(Hkv, D), pos, s.rope_theta))
    v = R((W.Wv[l] @ a).reshape(Hkv, D))
    o = np.empty((Hq, D))
    for hq in range(Hq):
        j = hq // G
        Kp, Vp = past(j)
        o[hq] = attend(q[hq], np.concatenate([Kp, k[j][None]]), np.concatenate([Vp, v[j][None]]))
    o = R(o)
    h = R(h + W.Wo[l] @ o.reshape(-1))
    f = R(rmsnorm(h, W.g2[l], s.eps))
    m = R(silu(W.W1[l] @ f) * (W.W3[l] @ f))
    h = R(h + W.W2[l] @ m)
    return h, k, v, q, o


def head_forward(W: Weights, h: np.ndarray, rdtype: str | None = None) -> np.ndarray:
    """Final norm and LM head of one row: float64 logits [V]."""
    R = storage_round(rdtype or W.dtype)
    return W.Wlm @ R(rmsnorm(h, W.gF, W.shape.eps))


def row_forward(W: Weights, tok: int, pos: int, past, rdtype: str | None = None) -> RowOut:
    """One token through the whole model.

    past(l, j) -> (K [n][D], V [n][D]): the cached rows visible to this row for
    layer l, KV head j, in absolute-position order (this row's own K/V is
    appended after them).  Returns float64 logits [V], this row's K/V rows
    [L][Hkv][D] (as stored) and its post-RoPE queries [L][Hq][D].
    """
    s = W.shape
    R = storage_round(rdtype or W.dtype)
    L, Hq, Hkv, D = s.n_layers, s.n_q_heads, s.n_kv_heads, s.head_dim
    ks = np.empty((L, Hkv, D))
    vs = np.empty((L, Hkv, D))
    qs = np.empty((L, Hq, D))
    h = R(W.E[tok])
    for l in range(L):
        h, ks[l], vs[l], qs[l], _ = layer_forward(W, l, h, pos, lambda j, l=l: past(l, j), rdtype)
    return RowOut(head_forward(W, h, rdtype), ks, vs, qs)


def argmax(logits: np.ndarray) -> int:
    """Greedy choice; ties go to the lowest index (np.argmax returns the first maximum)."""
    return int(np.argmax(logits))


def sequence_logits(W: Weights, tokens, rdtype: str | None = None) -> np.ndarray:
    """Brute-force reference with no cache: the whole sequence in matrix form,
    causal mask, every position's logits [n][V].  Written independently of
    row_forward (matrix attention, explicit mask) for the no-cache pin."""
    s = W.shape
    R = storage_round(rdtype or W.dtype)
    D, G, n = s.head_dim, s.group, len(tokens)
    Hq, Hkv = s.n_q_heads, s.n_kv_heads
    H = R(W.E[np.asarray(tokens)])                                   # [n][d]
    mask = np.tril(np.ones((n, n), dtype=bool))
    for l in range(s.n_layers):
        A = R(rmsnorm(H, W.g1[l], s.eps))
        Q = (A @ W.Wq[l].T).reshape(n, Hq, D)
        K = (A @ W.Wk[l].T).reshape(n, Hkv, D)
        V = R((A @ W.Wv[l].T).reshape(n, Hkv, D))
        Q = R(np.stack([rope(Q[p], p, s.rope_theta) for p in range(n)]))
        K = R(np.stack([rope(K[p], p, s.rope_theta) for p in range(n)]))
        O = np.empty((n, Hq, D))
        for hq in range(Hq):
            j = hq // G
            S = (Q[:, hq, :] @ K[:, j, :].T) / math.sqrt(D)
            S = np.where(mask, S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            O[:, hq, :] = P @ V[:, j, :]
        O = R(O)
        H = R(H + O.reshape(n, -1) @ W.Wo[l].T)
        F = R(rmsnorm(H, W.g2[l], s.eps))
        M = R(silu(F @ W.W1[l].T) * (F @ W.W3[l].T))
        H = R(H + M @ W.W2[l].T)
    Z = R(rmsnorm(H, W.gF, s.eps))
    return Z @ W.Wlm.T


# ---------------------------------------------------------------- full-size forms (8B shapes)
# At the 8B shapes the whole model does not fit in host memory as float64 (64 GB), and one row at
# a time against a 65536-row cache is slow.  These forms compute the same values as Weights,
# head_forward and layer_forward, one layer at a time; tests/test_oracle_model.py pins each to
# the form above on small shapes.

def _stored_chunked(stream: int, out_dim: int, in_dim: int, seed: int, dtype: str, pool, rows: int = 2048):
    """One [out][in] matrix of the Weights recipe, generated in row chunks (the draws are
    counter based: chunk r0 starts at element r0 * in_dim), possibly on a thread pool."""
    def chunk(r0):
        r1 = min(out_dim, r0 + rows)
        x = synth.xavier(stream, (r1 - r0, in_dim), in_dim, out_dim, seed, start=r0 * in_dim)
        return _stored(x, dtype)
    starts = range(0, out_dim, rows)
    parts = list(pool.map(chunk, starts)) if pool is not None else [chunk(r0) for r0 in starts]
    return np.concatenate(parts)


class LayerWeights:
    """Layer l's weights only, with the attribute layout of Weights (Wq[l], ..., g1[l]) so that
    layer_forward and layer_forward_rows take it in place of a whole model."""

    def __init__(self, shape: ModelShape, l: int, seed: int = 0, dtype: str | None = None, pool=None):
        s = shape
        dt = dtype or s.dtype
        self.shape, self.dtype = s, dt
        D = s.head_dim
        st = lambda t: synth.layer_stream(l, t)
        mat = lambda t, o, i: _stored_chunked(st(t), o, i, seed, dt, pool)
        self.Wq = {l: mat(synth.T_WQ, s.n_q_heads * D, s.d_model)}
        self.Wk = {l: mat(synth.T_WK, s.n_kv_heads * D, s.d_model)}
        self.Wv = {l: mat(synth.T_WV, s.n_kv_heads * D, s.d_model)}
        self.Wo = {l: mat(synth.T_WO, s.d_model, s.n_q_heads * D)}
        self.W1 = {l: mat(synth.T_W1, s.ffn, s.d_model)}
        self.W3 = {l: mat(synth.T_W3, s.ffn, s.d_model)}
        self.W2 = {l: mat(synth.T_W2, s.d_model, s.ffn)}
        self.g1 = {l: np.ones(s.d_model)}
        self.g2 = {l: np.ones(s.d_model)}


def embed_rows(shape: ModelShape, tokens, seed: int = 0, dtype: str | None = None) -> np.ndarray:
    """Rows E[tok] of the embedding (Weights.E), generated one row at a time."""
    s = shape
    dt = dtype or s.dtype
    return np.stack([_stored(synth.xavier(synth.S_EMBED, (1, s.d_model), s.d_model, s.vocab, seed,
                                          start=int(t) * s.d_model), dt)[0] for t in tokens])


def head_logits(shape: ModelShape, H: np.ndarray, seed: int = 0, dtype: str | None = None, pool=None,
                rows: int = 4096) -> np.ndarray:
    """head_forward for rows H [n][d]: final norm, then Wlm in row chunks -> logits [n][V]."""
    s = shape
    dt = dtype or s.dtype
    R = storage_round(dt)
    Z = R(rmsnorm(H, np.ones(s.d_model), s.eps))

    def chunk(r0):
        r1 = min(s.vocab, r0 + rows)
        Wc = _stored(synth.xavier(synth.S_LMHEAD, (r1 - r0, s.d_model), s.d_model, s.vocab, seed,
                                  start=r0 * s.d_model), dt)
        return Z @ Wc.T
    starts = range(0, s.vocab, rows)
    parts = list(pool.map(chunk, starts)) if pool is not None else [chunk(r0) for r0 in starts]
    return np.concatenate(parts, axis=1)


def layer_forward_rows(W, l: int, H: np.ndarray, pos0: int, Kp: np.ndarray, Vp: np.ndarray,
                       rdtype: str | None = None):
    """layer_forward for n consecutive rows at positions pos0 .. pos0 + n - 1 (residuals H [n][d]):
    row i sees the cached rows Kp, Vp [Hkv][T][D] and rows 0..i of this call, in absolute-position
    order.  The projections take all rows at once, and the G query heads of a KV head are scored
    against the cached rows together; every row's values are those of layer_forward (up to the
    order of float64 sums).  Returns (H_out [n][d], K [n][Hkv][D], V [n][Hkv][D])."""
    s = W.shape
    R = storage_round(rdtype or W.dtype)
    D, G, Hq, Hkv = s.head_dim, s.group, s.n_q_heads, s.n_kv_heads
    n = H.shape[0]
    A = R(rmsnorm(H, W.g1[l], s.eps))
    Q = A @ W.Wq[l].T
    Kn = A @ W.Wk[l].T
    Q = R(np.stack([rope(Q[i].reshape(Hq, D), pos0 + i, s.rope_theta) for i in range(n)]))     # [n][Hq][D]
    Kn = R(np.stack([rope(Kn[i].reshape(Hkv, D), pos0 + i, s.rope_theta) for i in range(n)]))  # [n][Hkv][D]
    Vn = R((A @ W.Wv[l].T).reshape(n, Hkv, D))
    O = np.empty((n, Hq, D))
    mask = np.repeat(np.tril(np.ones((n, n), dtype=bool)), G, axis=0)      # [(row, head)][row of this call]
    for j in range(Hkv):
        Qj = Q[:, j * G:(j + 1) * G, :].reshape(n * G, D)                  # (row, head) pairs
        Sc = (Qj @ Kp[j].T) / math.sqrt(D)                                  # against the cached rows
        Sn = np.where(mask, (Qj @ Kn[:, j, :].T) / math.sqrt(D), -np.inf)  # against this call's rows
        mx = np.maximum(Sc.max(axis=1), Sn.max(axis=1))[:, None]
        Pc, Pn = np.exp(Sc - mx), np.exp(Sn - mx)
        den = (Pc.sum(axis=1) + Pn.sum(axis=1))[:, None]
        O[:, j * G:(j + 1) * G, :] = ((Pc @ Vp[j] + Pn @ Vn[:, j, :]) / den).reshape(n, G, D)
    O = R(O)
    H = R(H + O.reshape(n, -1) @ W.Wo[l].T)
    F = R(rmsnorm(H, W.g2[l], s.eps))
    M = R(silu(F @ W.W1[l].T) * (F @ W.W3[l].T))
    H = R(H + M @ W.W2[l].T)
    return H, Kn, Vn
