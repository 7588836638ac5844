"""Sampled decoding for the oracle: a counter-based generator, tempered-softmax
sampling, and speculative rejection sampling over the VeriCache loop.
TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  [VC2] "VeriCache Guide: Lossless Inference with Lossy KV Caches", section
        "Mathematical Guarantee of Lossless Correctness": a candidate drawn
        from the draft distribution is kept with probability
        min(1, p_target(x) / p_draft(x)); after a rejection the replacement is
        drawn from max(0, p_target - p_draft) renormalised; the emitted token
        is then distributed exactly as p_target.
  [VC1] "VeriCache: Making Lossy KV Compression Exact", "Final Takeaways":
        sampled decoding needs machinery beyond the greedy exact-match rule.
  Philox4x64-10: Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
        Easy as 1, 2, 3" (SC 2011): ten rounds of two 64x64 -> 128-bit
        multiplies (multipliers 0xD2E7470EE14C6C93, 0xCA5A826395121157) with a
        Weyl key schedule (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B).

Readings where the pages are silent:
  - p = softmax(logits / temperature).  Temperature 0 means the one-hot
    distribution at the greedy choice (lowest index of the largest logit), so
    every rule below then reduces exactly to greedy VeriCache.
  - The verifier's distribution for draft i is that of verify row i (the row
    whose output predicts draft i's position); with all x drafts kept, the
    bonus token is drawn from verify row x.
  - The acceptance test is u * p_draft(x) < p_target(x) (no division).
  - Inverse-CDF sampling over non-negative weights: the smallest index whose
    running sum exceeds u * (total weight); if none does (only through
    rounding), the last index of positive weight.
  - A rejection whose residual has no positive mass (only through rounding)
    draws from p_target with the rejected candidate's weight set to zero, so
    that the emitted token always differs from the rejected draft.
  - A row whose logits hold NaN or +inf, or nothing finite, yields token -1.
  - Uniforms: key (seed, 0), counter (position, purpose, stream, 0), where
    position is the absolute position of the token being chosen and purpose
    is DRAFT, ACCEPT or TARGET; u = (first output word >> 40) / 2^24, a
    multiple of 2^-24 in [0, 1).  A round that rejects at i discards the
    drafts after i unseen, so the next round may draw those positions' DRAFT
    uniforms again: nothing emitted depended on them.

Parity: philox4x64_10 is pinned to numpy.random.Philox and to the published
all-zero known answer; the rejection rule by the exact marginal identity
(rational arithmetic) and by chi-square tests of emitted-token frequencies;
temperature 0 by equality with the greedy loops.
"""
from __future__ import annotations

import numpy as np

from .decode import Prefill, RoundLog, prefill
from .kvcache import RowStore, chain
from .model import Weights, argmax, row_forward

_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B
_MASK = (1 << 64) - 1

DRAFT, ACCEPT, TARGET = 0, 1, 2


def philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds: counter (4 words) and key (2 words) of 64
    bits -> 4 output words.  Each round multiplies words 0 and 2 by the two
    multipliers; the new words are (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2),
    hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)); the key advances by the Weyl constants
    between rounds."""
    x0, x1, x2, x3 = (int(c) & _MASK for c in ctr)
    k0, k1 = (int(k) & _MASK for k in key)
    for r in range(10):
        if r:
            k0, k1 = (k0 + _W0) & _MASK, (k1 + _W1) & _MASK
        p0, p1 = _M0 * x0, _M1 * x2
        x0, x1, x2, x3 = ((p1 >> 64) ^ x1 ^ k0) & _MASK, p1 & _MASK, ((p0 >> 64) ^ x3 ^ k1) & _MASK, p0 & _MASK
    return x0, x1, x2, x3


def uniform(seed: int, stream: int, pos: int, purpose: int) -> float:
    """The draw of (stream, position, purpose): a multiple of 2^-24 in [0, 1)."""
    r = philox4x64_10((pos, purpose, stream, 0), (seed, 0))[0]
    return (r >> 40) / float(1 << 24)


def tempered_probs(logits, tau: float):
    """softmax(logits / tau) in float64, or None for a row with NaN, +inf or
    nothing finite; tau == 0 gives the one-hot row at the greedy argmax."""
    z = np.asarray(logits, dtype=np.float64)
    if np.isnan(z).any() or np.isposinf(z).any() or not np.isfinite(z).any():
        return None
    if tau == 0:
        p = np.zeros(z.shape)
        p[argmax(z)] = 1.0
        return p
    w = np.exp((z - z.max()) / tau)
    return w / w.sum()


def sample_index(w, u: float):
    """Inverse-CDF draw from non-negative weights w (any scale) with u in
    [0, 1).  Returns (index, margin): margin is the distance of u * sum(w)
    from the nearest edge of the chosen index's interval, over sum(w) (how
    far the draw was from choosing a neighbour)."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    total = c[-1]
    target = u * total
    hit = np.nonzero(c > target)[0]
    if len(hit) == 0:
        k = int(np.nonzero(w > 0)[0][-1])
        return k, 0.0
    k = int(hit[0])
    lo = c[k - 1] if k else 0.0
    return k, float(min(target - lo, c[k] - target) / total)


def accept_probability(pt, pd, x: int):
    """min(1, p_target(x) / p_draft(x)) for a candidate x drawn from p_draft
    (so p_draft(x) > 0); plain arithmetic, so it also runs on Fractions."""
    return min(1, pt[x] / pd[x])


def residual(pt, pd):
    """max(0, p_target - p_draft) renormalised (None when it has no mass);
    plain arithmetic, so it also runs on Fractions."""
    r = [max(0, a - b) for a, b in zip(pt, pd)]
    s = sum(r)
    if s == 0:
        return None
    return [v / s for v in r]


def residual_weights(pt, pd):
    """max(0, p_target - p_draft) elementwise, unnormalised (float64 arrays)."""
    return np.maximum(0.0, np.asarray(pt, dtype=np.float64) - np.asarray(pd, dtype=np.float64))


def speculative_accept(pt_rows, pd_rows, draft, u_acc, u_res):
    """One round of speculative rejection sampling.

    pt_rows: x + 1 target distributions (verify rows 0..x); pd_rows: x draft
    distributions; draft: the x drafted tokens; u_acc[i]: the acceptance draw
    of draft i; u_res[i]: the draw that chooses the token of row i when row i
    is the first rejection (i < x) or the bonus (i = x).  Returns (a, token,
    margins): a drafts kept, the token emitted after them, and the margins of
    every decision taken (acceptance tests: |u p_d - p_t| / max(p_d, p_t);
    the final draw: sample_index's margin)."""
    x = len(draft)
    margins = []
    for i in range(x):
        pt, pd, d = pt_rows[i], pd_rows[i], int(draft[i])
        lhs, rhs = u_acc[i] * pd[d], pt[d]
        margins.append(abs(lhs - rhs) / max(pd[d], pt[d], 1e-300))
        if lhs < rhs:
            continue
        r = residual_weights(pt, pd)
        if not r.sum() > 0:
            r = np.array(pt, dtype=np.float64)
            r[d] = 0.0
        k, m = sample_index(r, u_res[i])
        margins.append(m)
        return i, k, margins
    k, m = sample_index(pt_rows[x], u_res[x])
    margins.append(m)
    return x, k, margins


def sample_row(logits, tau: float, seed: int, stream: int, pos: int, purpose: int):
    """The token chosen at position pos from one logits row: (token, margin,
    probabilities or None)."""
    p = tempered_probs(logits, tau)
    if p is None:
        return -1, 0.0, None
    k, m = sample_index(p, uniform(seed, stream, pos, purpose))
    return k, m, p


def sampled_decode(W: Weights, prompt, n_tokens: int, tau: float, seed: int, stream: int = 0,
                   pre: Prefill | None = None):
    """Full-KV sampled decoding: the token at position p is drawn from the
    target distribution of the row before it with the TARGET draw of p.
    Returns (tokens, margins)."""
    pre = pre or prefill(W, prompt)
    full = pre.full.copy()
    T = len(prompt)
    g0, m0, _ = sample_row(pre.last_logits, tau, seed, stream, T, TARGET)
    toks, margins = [g0], [m0]
    while len(toks) < n_tokens:
        p = T + len(toks)
        out = row_forward(W, toks[-1], p - 1, full.rows)
        full.append(out.k, out.v)
        t, m, _ = sample_row(out.logits, tau, seed, stream, p, TARGET)
        toks.append(t)
        margins.append(m)
    return toks, margins


class SampledRound(RoundLog):
    """A round of sampled VeriCache: RoundLog's fields (verified = the tokens
    the verifier's decisions imply: the kept drafts, then the emitted token)
    plus the margins of every draw and test the round took."""
    __slots__ = ("margins",)


def vericache_sampled(W: Weights, prompt, n_tokens: int, x: int, make_draft_cache, tau: float, seed: int,
                      stream: int = 0, pre: Prefill | None = None):
    """The VeriCache loop with sampled drafts and speculative rejection
    sampling in place of exact-match acceptance.  g0 is drawn from the
    prefill's last row.  Each round: draft i (position pos + 1 + i) is drawn
    from the compressed-cache distribution with the DRAFT draw of its
    position; the x + 1 verify rows give the target distributions; the
    acceptance tests use the ACCEPT draws and the final token the TARGET draw
    of its position.  The verifier's K/V rows 0..a are committed as in the
    greedy loop.  Returns (tokens, rounds)."""
    s = W.shape
    pre = pre or prefill(W, prompt)
    full = pre.full.copy()
    comp = make_draft_cache(pre)
    tail = RowStore(s.n_layers, s.n_kv_heads, s.head_dim)
    T = len(prompt)
    g0, _, _ = sample_row(pre.last_logits, tau, seed, stream, T, TARGET)
    out = [g0]
    pending, pos = g0, T
    rounds = []
    while len(out) < n_tokens:
        if pending < 0:
            raise FloatingPointError("non-finite logits")
        dtail = RowStore(s.n_layers, s.n_kv_heads, s.head_dim)
        past = chain(comp, tail, dtail)
        draft, pd_rows, margins, t = [], [], [], pending
        for i in range(x):
            o = row_forward(W, t, pos + i, past)
            dtail.append(o.k, o.v)
            t, m, p = sample_row(o.logits, tau, seed, stream, pos + 1 + i, DRAFT)
            if t < 0:
                raise FloatingPointError("non-finite draft logits")
            draft.append(t)
            pd_rows.append(p)
            margins.append(m)
        rows = [pending] + draft
        vrows = RowStore(s.n_layers, s.n_kv_heads, s.head_dim)
        vpast = chain(full, vrows)
        pt_rows, kv = [], []
        for i, tok in enumerate(rows):
            o = row_forward(W, tok, pos + i, vpast)
            vrows.append(o.k, o.v)
            kv.append((o.k, o.v))
            pt = tempered_probs(o.logits, tau)
            if pt is None:
                raise FloatingPointError("non-finite verify logits")
            pt_rows.append(pt)
        u_acc = [uniform(seed, stream, pos + 1 + i, ACCEPT) for i in range(x)]
        u_res = [uniform(seed, stream, pos + 1 + i, TARGET) for i in range(x + 1)]
        a, tok, m2 = speculative_accept(pt_rows, pd_rows, draft, u_acc, u_res)
        emitted = draft[:a] + [tok]
        r = SampledRound(pos, draft, draft[:a] + [tok], a, emitted)
        r.margins = margins + m2
        rounds.append(r)
        out += emitted
        for i in range(a + 1):
            full.append(*kv[i])
            tail.append(*kv[i])
        pending, pos = tok, pos + a + 1
    return out[:n_tokens], rounds
