"""Oracle decode loops: full-KV greedy and the VeriCache draft / verify / accept loop.

Greedy ([KV4] "Autoregressive Decoding and the KV Cache"): prefill the prompt
at positions 0..T-1, emit g0 = argmax of row T-1, then g_i = argmax of the
row for g_{i-1} at position T+i-1.  N emitted tokens include g0.

VeriCache round ([VC1] "The Core Idea", pseudocode and worked example;
[VC3] "实践案例" case 1):
    rows    = [pending] + draft            pending = last emitted token, not yet in any cache
    draft   : x greedy steps over the draft cache (compressed rows + committed
              exact rows + this round's own draft rows)
    verify  : the x + 1 rows at positions pos..pos+x, each seeing the full KV and
              the verify rows before it; ver[i] = argmax of row i
              (ver[0..x-1] check the drafts, ver[x] is the bonus prediction)
    accept  : a = first i with draft[i] != ver[i], else x
    emit    : draft[:a] + [ver[a]]          (a + 1 tokens; x + 1 when every draft matched)
    commit  : the verifier's exact K/V rows 0..a (pending, draft[0..a-1]) are
              appended to the full KV and to the draft cache's exact tail;
              draft rows are discarded; pending = ver[a]; pos += a + 1
Readings where the pages are silent:
    - the verifier's rows, not the draft's, are what the caches keep for accepted tokens;
    - generated rows are never re-compressed: the tail stays in the model dtype;
    - every round drafts a full x, and the output is cut to N at the end;
    - the acceptance rule here is greedy exact match; sampled decoding with
      speculative rejection sampling is in sampling.py.
"""
from __future__ import annotations

import math

import numpy as np

from .compress import Quantized, tokdrop, tokdrop_keynorm
from .kvcache import FixedRows, RowStore, chain
from .model import Weights, argmax, head_forward, rmsnorm, rope, row_forward, silu, storage_round


def accept(draft, verified):
    """Accept-until-first-mismatch ([VC1] "The Core Idea").

    draft has x tokens, verified has x + 1 predictions.  Returns (a, emitted):
    a = number of leading drafts equal to the verifier's predictions, emitted
    = draft[:a] + [verified[a]] (the correction at a mismatch, the bonus token
    when a == x).
    """
    x = len(draft)
    assert len(verified) == x + 1
    a = x
    for i in range(x):
        if draft[i] != verified[i]:
            a = i
            break
    return a, list(draft[:a]) + [verified[a]]


class Prefill:
    __slots__ = ("full", "g0", "q_obs", "last_logits")

    def __init__(self, full, g0, q_obs, last_logits):
        self.full, self.g0, self.q_obs, self.last_logits = full, g0, q_obs, last_logits


def prefill(W: Weights, prompt, obs_window: int = 32) -> Prefill:
    """Rows 0..T-1 one at a time; keeps the post-RoPE queries of the last
    obs_window positions ([L][Hq][W][D]) for the token-drop compressor."""
    s = W.shape
    T = len(prompt)
    full = RowStore(s.n_layers, s.n_kv_heads, s.head_dim, max(T, 1))
    wn = min(obs_window, T)
    q_obs = np.zeros((s.n_layers, s.n_q_heads, wn, s.head_dim))
    out = None
    for p, tok in enumerate(prompt):
        out = row_forward(W, int(tok), p, full.rows)
        full.append(out.k, out.v)
        if p >= T - wn:
            q_obs[:, :, p - (T - wn)] = out.q
    return Prefill(full, argmax(out.logits), q_obs, out.logits)


def prefill_matrix(W: Weights, prompt, obs_window: int = 32) -> Prefill:
    """prefill() in matrix form: each layer over all prompt rows at once (causal mask), with the
    rounding points of layer_forward, for long prompts at large widths.  The stored values equal
    the row-at-a-time prefill's up to float64 summation order (pinned against it)."""
    s = W.shape
    R = storage_round(W.dtype)
    L, Hq, Hkv, D, G = s.n_layers, s.n_q_heads, s.n_kv_heads, s.head_dim, s.group
    toks = np.asarray(prompt, dtype=np.int64)
    n = len(toks)
    wn = min(obs_window, n)
    full = RowStore(L, Hkv, D, max(n, 1))
    q_obs = np.zeros((L, Hq, wn, D))
    mask = np.tril(np.ones((n, n), dtype=bool))
    H = R(W.E[toks])
    for l in range(L):
        A = R(rmsnorm(H, W.g1[l], s.eps))
        Q = R(np.stack([rope(q, p, s.rope_theta) for p, q in enumerate((A @ W.Wq[l].T).reshape(n, Hq, D))]))
        K = R(np.stack([rope(k, p, s.rope_theta) for p, k in enumerate((A @ W.Wk[l].T).reshape(n, Hkv, D))]))
        V = R((A @ W.Wv[l].T).reshape(n, Hkv, D))
        O = np.empty((n, Hq, D))
        for hq in range(Hq):
            j = hq // G
            S = np.where(mask, (Q[:, hq] @ K[:, j].T) / math.sqrt(D), -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            O[:, hq] = (P / P.sum(axis=1, keepdims=True)) @ V[:, j]
        O = R(O)
        H = R(H + O.reshape(n, -1) @ W.Wo[l].T)
        F = R(rmsnorm(H, W.g2[l], s.eps))
        M = R(silu(F @ W.W1[l].T) * (F @ W.W3[l].T))
        H = R(H + M @ W.W2[l].T)
        full.K[l, :, :n] = K.transpose(1, 0, 2)
        full.V[l, :, :n] = V.transpose(1, 0, 2)
        q_obs[l] = Q[n - wn:].transpose(1, 0, 2)
    full.n = n
    last = head_forward(W, H[-1])
    return Prefill(full, argmax(last), q_obs, last)


def greedy(W: Weights, prompt, n_tokens: int, pre: Prefill | None = None, force=None):
    """Full-KV greedy decode.  Returns (tokens, per-step logits).

    force: optional token list; step i then consumes force[i-1] instead of the
    model's own choice (teacher forcing after a flagged near-tie divergence)."""
    pre = pre or prefill(W, prompt)
    full = pre.full.copy()
    T = len(prompt)
    toks = [pre.g0]
    logits = [pre.last_logits]
    while len(toks) < n_tokens:
        i = len(toks)
        prev = toks[-1] if force is None else int(force[i - 1])
        out = row_forward(W, prev, T + i - 1, full.rows)
        full.append(out.k, out.v)
        toks.append(argmax(out.logits))
        logits.append(out.logits)
    return toks, logits


# --------------------------------------------------------------------------
# draft caches built from the prefill
# --------------------------------------------------------------------------
def draft_cache_identity(pre: Prefill, **_):
    """No compression: the draft cache equals the full prefill KV (every round then
    accepts all x drafts; used to pin the bonus-token rule)."""
    return pre.full.copy()


def draft_cache_tokdrop(pre: Prefill, W: Weights, keep_total: int, keep_recent: int = 64, **_):
    L, H = W.shape.n_layers, W.shape.n_kv_heads
    n = pre.full.n
    Kf = pre.full.K[:, :, :n]
    Vf = pre.full.V[:, :, :n]
    idx, Kk, Vk, _scores = tokdrop(Kf, Vf, pre.q_obs, keep_total, keep_recent, W.shape.group)
    return FixedRows([[Kk[l, j] for j in range(H)] for l in range(L)],
                     [[Vk[l, j] for j in range(H)] for l in range(L)])


def draft_cache_keynorm(pre: Prefill, W: Weights, keep_total: int, **_):
    """Token drop ranked by key norm: per layer, the keep_total prompt rows of largest mean key
    norm over the KV heads ([VC2] "The Uniform Compressor Interface")."""
    L, H = W.shape.n_layers, W.shape.n_kv_heads
    n = pre.full.n
    idx, Kk, Vk, _scores = tokdrop_keynorm(pre.full.K[:, :, :n], pre.full.V[:, :, :n], keep_total)
    return FixedRows([[Kk[l, j] for j in range(H)] for l in range(L)],
                     [[Vk[l, j] for j in range(H)] for l in range(L)])


def draft_cache_quant(pre: Prefill, W: Weights, bits: int, group: int, **_):
    n = pre.full.n
    q = Quantized(pre.full.K[:, :, :n], pre.full.V[:, :, :n], bits, group)
    Kd, Vd = q.rows_K(), q.rows_V()
    L, H = Kd.shape[:2]
    return FixedRows([[Kd[l, j] for j in range(H)] for l in range(L)],
                     [[Vd[l, j] for j in range(H)] for l in range(L)])


def rel_gap(logits: np.ndarray) -> float:
    """(top-1 - top-2) / max |logit|: how far a greedy choice is from a tie, relative to the
    logits' scale (positions below a comparison tolerance are near-ties)."""
    srt = np.sort(np.asarray(logits))[::-1]
    return float((srt[0] - srt[1]) / max(np.abs(srt).max(), 1e-300))


class RoundLog:
    """One round: position of the pending token, drafts, verifier's predictions, accept count,
    emitted tokens, and the relative top-2 gaps of every draft and verify row."""
    __slots__ = ("pos", "draft", "verified", "a", "emitted", "draft_gap", "verify_gap")

    def __init__(self, pos, draft, verified, a, emitted, draft_gap=None, verify_gap=None):
        self.pos, self.draft, self.verified, self.a, self.emitted = pos, draft, verified, a, emitted
        self.draft_gap, self.verify_gap = draft_gap, verify_gap


class DraftLength:
    """Draft length per round, with a fall back to plain decoding.

    [VC3] "踩过的坑": a short verification cycle wastes the long accepted runs,
    so x should grow with the acceptance; [KV4] "When the Serving Stack Breaks
    Down": when drafts stop matching, speculation costs a draft pass and a
    verification pass for the one token plain decoding would give, so fall
    back to plain decoding.  Reading (the pages give no numbers): start at
    x_max; after a round that keeps all x drafts, double x (at most x_max);
    after a rejection at a, x = max(x_min, a + 1); after fallback_after
    consecutive rounds that keep no draft (0: never), decode plainly (x = 0:
    the round verifies the pending token alone and emits one token) for
    plain_rounds rounds, then probe again at x_min.  The tokens do not depend
    on any of this (every x gives the greedy tokens), only the work per token.
    """

    def __init__(self, x_max: int, x_min: int = 1, fallback_after: int = 0, plain_rounds: int = 8):
        self.x_max, self.x_min = x_max, max(1, min(x_min, x_max))
        self.fallback_after, self.plain_rounds = fallback_after, plain_rounds
        self.x = x_max
        self.zero_run = 0
        self.plain_left = 0

    def after(self, a: int) -> None:
        if self.x == 0:
            self.plain_left -= 1
            if self.plain_left <= 0:
                self.x, self.zero_run = self.x_min, 0
            return
        self.zero_run = self.zero_run + 1 if a == 0 else 0
        if self.fallback_after and self.zero_run >= self.fallback_after:
            self.x, self.plain_left = 0, self.plain_rounds
        elif a == self.x:
            self.x = min(self.x_max, 2 * self.x)
        else:
            self.x = max(self.x_min, a + 1)


def vericache(W: Weights, prompt, n_tokens: int, x: int, make_draft_cache, pre: Prefill | None = None,
              drafter=None, policy: DraftLength | None = None):
    """The VeriCache loop.  Returns (tokens, rounds).

    make_draft_cache(pre) -> segment with rows(l, j) (the compressed cache).
    drafter(round_index, pending, own_draft) -> replacement draft list (to test
        that any drafter still yields the greedy output); None keeps the model's drafts.
    policy: a DraftLength choosing each round's x (None: x every round).
    """
    s = W.shape
    pre = pre or prefill(W, prompt)
    full = pre.full.copy()
    comp = make_draft_cache(pre)
    tail = RowStore(s.n_layers, s.n_kv_heads, s.head_dim)
    T = len(prompt)
    out = [pre.g0]
    pending, pos = pre.g0, T
    rounds = []
    while len(out) < n_tokens:
        # ---- draft x tokens with the compressed cache
        dtail = RowStore(s.n_layers, s.n_kv_heads, s.head_dim)
        past = chain(comp, tail, dtail)
        xr = x if policy is None else policy.x
        draft, t, dgap = [], pending, []
        for i in range(xr):
            o = row_forward(W, t, pos + i, past)
            dtail.append(o.k, o.v)
            t = argmax(o.logits)
            draft.append(t)
            dgap.append(rel_gap(o.logits))
        if drafter is not None:
            draft = [int(v) for v in drafter(len(rounds), pending, draft)]
        # ---- verify x + 1 rows against the full KV
        rows = [pending] + draft
        vrows = RowStore(s.n_layers, s.n_kv_heads, s.head_dim)
        vpast = chain(full, vrows)
        ver, kv, vgap = [], [], []
        for i, tok in enumerate(rows):
            o = row_forward(W, tok, pos + i, vpast)
            vrows.append(o.k, o.v)
            kv.append((o.k, o.v))
            ver.append(argmax(o.logits))
            vgap.append(rel_gap(o.logits))
        # ---- accept and commit
        a, emitted = accept(draft, ver)
        rounds.append(RoundLog(pos, draft, ver, a, emitted, dgap, vgap))
        if policy is not None:
            policy.after(a)
        out += emitted
        for i in range(a + 1):
            full.append(*kv[i])
            tail.append(*kv[i])
        pending, pos = out[-1], pos + a + 1
    return out[:n_tokens], rounds
