"""Oracle compressors: what compress(full_k, full_v) produces ([VC2] "The Uniform
Compressor Interface"; its prototype keeps top-k indices and sorts them
ascending before gathering).

Two families, run per layer l and per KV head j on the prefill's K (after
RoPE) and V:

Token drop by observed attention (SnapKV-like; the rule of the token-drop workloads)
    W observation queries (the last W prompt positions), R recent rows, keep K rows.
    p[h,i,t] = softmax over t' <= i of q[h,i] . k[t'] / sqrt(D)  for h in the
               GQA group of j and i in [T-W, T)
    s[t]     = mean over (h, i) of p[h,i,t], for candidates t < T - R
    keep     = top-(K - R) candidates by s (ties: smaller t), plus [T-R, T), ascending.
    If every candidate fits, nothing is dropped.

Token drop by key norm ([VC2] "The Uniform Compressor Interface": its example
compressor ranks tokens by key energy)
    per layer l: e[t] = mean over the KV heads j of ||k[l,j,t]||_2 (one ranking shared by
    every head of the layer); keep = the max(32, T // ratio) tokens of largest e (ties:
    smaller t), ascending; no recent window.  If every token fits, nothing is dropped.

Per-group asymmetric quantization (KIVI-style: K per channel, V per token)
    b in {2,3,4}, group G, Tq = floor(T/G)*G; rows [Tq, T) stay unquantized.
    For each group, in IEEE float32:
        mn, mx   = min, max
        zero     = fp16(mn)
        scale    = fp16((mx - mn) / (2^b - 1))
        code     = 0 if scale == 0 else clamp(rint((x - zero) / scale), 0, 2^b - 1)
    dequantized value = code * scale + zero (exact in float64).
    The pages give only "fp16 scale and zero"; min/max with zero = min,
    round-half-even codes and an IEEE divide are the plain reading.

Packed layout (byte-exact contract with the GPU compressor; every section
starts at a multiple of 256 bytes):
    quant:   Kc  [L][Hkv][Tq][D*b/8]        u8   token rows, code of channel d at bits [d*b, d*b+b)
             Vc  [L][Hkv][Tq/64][D][64*b/8] u8   per channel, 64 consecutive tokens, token i at bits [i*b, i*b+b)
             Ks  [L][Hkv][Tq/G][D]          fp16 scale;  Kz same shape: zero
             Vs  [L][Hkv][Tq][D/G]          fp16 scale;  Vz same shape: zero
             Kr  [L][Hkv][T-Tq][D], Vr same  residual rows in the model dtype
    tokdrop: Kk  [L][Hkv][Kk][D], Vk same (model dtype), idx [L][Hkv][Kk] int32 ascending
Bitstreams are little-endian: stream bit n is bit (n mod 8) of byte floor(n/8).

Pins (tests/test_oracle_compress.py): constant groups, exactly representable
ramps, the reconstruction bound, brute-force nearest-code search, a literal
packed-byte fixture, T <= K keeping everything, one-hot crafted attention
giving a known keep set, and a brute-force full sort for the top-k; for the
key-norm ranking, keys of known norms, heads that disagree (the mean decides),
a per-token norm recomputed by a plain loop, and the shared per-layer set.
"""
from __future__ import annotations

import math

import numpy as np

ALIGN = 256


def _align(n: int) -> int:
    return (n + ALIGN - 1) // ALIGN * ALIGN


# --------------------------------------------------------------------------
# token drop
# --------------------------------------------------------------------------
def tokdrop_scores(q_obs: np.ndarray, K: np.ndarray, n_cand: int) -> np.ndarray:
    """q_obs [G][W][D] (the GQA group's queries at positions T-W..T-1), K [T][D].
    Returns s [n_cand]: mean over (h, i) of the causal softmax probability of key t."""
    G, Wn, D = q_obs.shape
    T = K.shape[0]
    acc = np.zeros(n_cand)
    for h in range(G):
        for w in range(Wn):
            i = T - Wn + w
            sc = K[: i + 1] @ q_obs[h, w] / math.sqrt(D)
            p = np.exp(sc - sc.max())
            p /= p.sum()
            m = min(n_cand, i + 1)
            acc[:m] += p[:m]
    return acc / (G * Wn)


def tokdrop_select(scores: np.ndarray, T: int, keep_total: int, keep_recent: int) -> np.ndarray:
    """Kept positions, ascending: top-(keep_total - recent) candidates (ties to the
    smaller index) plus the recent window."""
    n_recent = min(keep_recent, T)
    n_cand = T - n_recent
    n_top = max(keep_total - n_recent, 0)
    if n_top >= n_cand:
        return np.arange(T, dtype=np.int32)
    order = np.lexsort((np.arange(n_cand), -scores[:n_cand]))   # primary: score desc, then index asc
    top = np.sort(order[:n_top])
    return np.concatenate([top, np.arange(n_cand, T)]).astype(np.int32)


def tokdrop(Kf: np.ndarray, Vf: np.ndarray, q_obs: np.ndarray, keep_total: int, keep_recent: int,
            group: int):
    """Kf, Vf [L][Hkv][T][D]; q_obs [L][Hq][W][D].  Returns (idx [L][Hkv][Kk], Kk, Vk, scores)."""
    L, H, T, D = Kf.shape
    n_recent = min(keep_recent, T)
    idx, scores = [], []
    for l in range(L):
        idx.append([])
        scores.append([])
        for j in range(H):
            s = tokdrop_scores(q_obs[l, j * group:(j + 1) * group], Kf[l, j], T - n_recent)
            idx[l].append(tokdrop_select(s, T, keep_total, keep_recent))
            scores[l].append(s)
    idx = np.asarray(idx, dtype=np.int32)
    Kk = np.take_along_axis(Kf, idx[..., None].astype(np.int64), axis=2)
    Vk = np.take_along_axis(Vf, idx[..., None].astype(np.int64), axis=2)
    return idx, Kk, Vk, scores


def keynorm_scores(K: np.ndarray) -> np.ndarray:
    """K [Hkv][T][D] of one layer.  e[t] = mean over heads of the L2 norm of key t."""
    K = np.asarray(K, dtype=np.float64)
    return np.sqrt((K * K).sum(axis=-1)).mean(axis=0)


def tokdrop_keynorm(Kf: np.ndarray, Vf: np.ndarray, keep_total: int):
    """Kf, Vf [L][Hkv][T][D].  Returns (idx [L][Hkv][Kk], Kk, Vk, scores [L][T]): per layer
    the top-keep_total tokens by key norm (ties to the smaller index), ascending, the same
    positions for every KV head of the layer."""
    L, H, T, D = Kf.shape
    idx, scores = [], []
    for l in range(L):
        e = keynorm_scores(Kf[l])
        sel = tokdrop_select(e, T, keep_total, 0)
        idx.append([sel] * H)
        scores.append(e)
    idx = np.asarray(idx, dtype=np.int32)
    Kk = np.take_along_axis(Kf, idx[..., None].astype(np.int64), axis=2)
    Vk = np.take_along_axis(Vf, idx[..., None].astype(np.int64), axis=2)
    return idx, Kk, Vk, np.asarray(scores)


# --------------------------------------------------------------------------
# quantization
# --------------------------------------------------------------------------
def quant_groups(x: np.ndarray, bits: int):
    """x [..., G] float32 values (each last-axis row is one group).
    Returns (codes uint8 [..., G], scale fp16 [...], zero fp16 [...])."""
    x = np.asarray(x, dtype=np.float32)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    zero = mn.astype(np.float16)
    scale = ((mx - mn) / np.float32(2 ** bits - 1)).astype(np.float16)   # float32 ops, then RNE to fp16
    z32 = zero.astype(np.float32)[..., None]
    s32 = scale.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.rint((x - z32) / s32)                                       # float32 subtract, divide, rint
    codes = np.where(s32 == 0, np.float32(0), np.clip(t, 0, 2 ** bits - 1))
    return codes.astype(np.uint8), scale, zero


def dequant(codes, scale, zero) -> np.ndarray:
    return codes.astype(np.float64) * scale.astype(np.float64)[..., None] + zero.astype(np.float64)[..., None]


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """Little-endian bitstream over the last axis: code n at stream bits [n*b, n*b+b)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    assert (n * bits) % 8 == 0
    bitarr = ((codes[..., None] >> np.arange(bits, dtype=np.uint8)) & 1).astype(np.uint8)
    bitarr = bitarr.reshape(codes.shape[:-1] + (n * bits,))
    return np.packbits(bitarr, axis=-1, bitorder="little")


def unpack_bits(packed: np.ndarray, bits: int, n: int) -> np.ndarray:
    b = np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=-1, bitorder="little")
    b = b[..., : n * bits].reshape(packed.shape[:-1] + (n, bits)).astype(np.uint8)
    return (b << np.arange(bits, dtype=np.uint8)).sum(axis=-1).astype(np.uint8)


class Quantized:
    """Per-request quantized cache, unpacked form plus dequantized float64 rows."""

    def __init__(self, Kf, Vf, bits, group):
        Kf = np.asarray(Kf, dtype=np.float32)
        Vf = np.asarray(Vf, dtype=np.float32)
        L, H, T, D = Kf.shape
        assert D % group == 0
        Tq = T // group * group
        ng = Tq // group
        self.bits, self.group, self.T, self.Tq = bits, group, T, Tq
        # K: per channel, groups of G consecutive tokens -> reshape [L][H][ng][G][D] -> group axis last
        kg = Kf[:, :, :Tq].reshape(L, H, ng, group, D).transpose(0, 1, 2, 4, 3)      # [L][H][ng][D][G]
        kc, self.ks, self.kz = quant_groups(kg, bits)                                  # ks [L][H][ng][D]
        self.kcodes = kc.transpose(0, 1, 2, 4, 3).reshape(L, H, Tq, D)                # [L][H][Tq][D]
        # V: per token, groups of G consecutive channels
        vg = Vf[:, :, :Tq].reshape(L, H, Tq, D // group, group)
        vc, self.vs, self.vz = quant_groups(vg, bits)                                  # vs [L][H][Tq][D/G]
        self.vcodes = vc.reshape(L, H, Tq, D)
        self.Khat = dequant(kc, self.ks, self.kz).transpose(0, 1, 2, 4, 3).reshape(L, H, Tq, D)
        self.Vhat = dequant(vc, self.vs, self.vz).reshape(L, H, Tq, D)
        self.Kres = Kf[:, :, Tq:].astype(np.float64)
        self.Vres = Vf[:, :, Tq:].astype(np.float64)

    def rows_K(self):
        """Draft-cache keys: dequantized [0, Tq) then residual [Tq, T)."""
        return np.concatenate([self.Khat, self.Kres], axis=2)

    def rows_V(self):
        return np.concatenate([self.Vhat, self.Vres], axis=2)


def quant_blob(q: Quantized, res_dtype: str) -> bytes:
    """Serialise a Quantized cache in the packed layout described in the module docstring."""
    L, H, Tq, D = q.kcodes.shape
    b = q.bits
    kc = pack_bits(q.kcodes, b)                                                    # [L][H][Tq][D*b/8]
    vblk = q.vcodes.reshape(L, H, Tq // 64, 64, D).transpose(0, 1, 2, 4, 3)       # [L][H][nb][D][64]
    vc = pack_bits(vblk, b)                                                        # [L][H][nb][D][8b]
    res = [_rows_bytes(q.Kres, res_dtype), _rows_bytes(q.Vres, res_dtype)]
    sections = [kc.tobytes(), vc.tobytes(), q.ks.astype("<f2").tobytes(), q.kz.astype("<f2").tobytes(),
                q.vs.astype("<f2").tobytes(), q.vz.astype("<f2").tobytes()] + res
    return _concat_aligned(sections)


def quant_sizes(L, H, T, D, bits, group, res_elem_bytes):
    """Section byte sizes of the quant layout, in order."""
    Tq = T // group * group
    ng = Tq // group
    return [L * H * Tq * D * bits // 8, L * H * Tq * D * bits // 8, L * H * ng * D * 2, L * H * ng * D * 2,
            L * H * Tq * (D // group) * 2, L * H * Tq * (D // group) * 2,
            L * H * (T - Tq) * D * res_elem_bytes, L * H * (T - Tq) * D * res_elem_bytes]


def tokdrop_blob(idx, Kk, Vk, dtype: str) -> bytes:
    return _concat_aligned([_rows_bytes(Kk, dtype), _rows_bytes(Vk, dtype),
                            np.asarray(idx, dtype="<i4").tobytes()])


def _rows_bytes(x: np.ndarray, dtype: str) -> bytes:
    x = np.asarray(x, dtype=np.float64)
    if dtype == "fp32":
        return x.astype("<f4").tobytes()
    # bf16: the values are already bf16-representable; take the top 16 bits of the float32 pattern
    u = x.astype(np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "row values are not bf16-representable"
    return (u >> 16).astype("<u2").tobytes()


def _concat_aligned(sections) -> bytes:
    out = bytearray()
    for s in sections:
        out += s
        out += b"\0" * (_align(len(out)) - len(out))
    return bytes(out)
