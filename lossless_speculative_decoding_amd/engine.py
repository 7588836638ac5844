"""Host-side VeriCache scheduler over the C ABI.

Per request ("Verifying Without Giving Back the Speedup", VeriCache: Making
Lossy KV Compression Exact): the compressed cache and a tail of exact rows
stay on the GPU; the rest of the full cache lives in pinned host memory and is
staged into one of the device slots (three by default) on a copy stream only for verification.
Rows the GPU already holds exactly (the committed tail, and the kept prompt
rows of a token-drop cache) are not kept on the host and never cross PCIe.  Requests
start drafting at staggered ticks (request r joins after floor(r * x / B)
ticks, the study note's "10 requests, x = 30: one verification every 3 draft
rounds"), so one request's transfer and verification overlap the others'
drafting.  A request's staging is issued `lead` ticks before its draft ends,
lead = ceil(t_copy / t_tick) (the guide's drafting-horizon sizing rule; by default
as soon as its drafting has begun, since one copy outlasts a round of drafts here);
verification never blocks the compute stream on a copy: the host polls the
copy event and keeps drafting other requests until the slot is ready.

All arithmetic runs in libvc.so; this module only sequences calls, owns the
buffers (torch allocations) and moves token ids it has already received.
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import time
from dataclasses import dataclass, field

import torch

import synth

from . import binding as B
from . import runtime
from ._vc import Req

DRAFT, WAIT_SLOT, ACCEPTING, DONE = range(4)


class NonFiniteLogits(RuntimeError):
    """The library wrote token -1: some row's logits had no finite maximum."""


def make_weights(shape, device="cuda", seed: int = 0) -> dict:
    """Random-init weights in the library layout, generated on the GPU from the
    seeded recipe (Xavier-uniform; norm gains 1)."""
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    L, d, Hq, Hkv, D, F, V = (shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                              shape.ffn, shape.vocab)
    e = lambda *sh: torch.empty(*sh, dtype=dt, device=device)
    W = {"embed": e(V, d), "lm_head": e(V, d), "norm_final": e(d), "norm_attn": e(L, d), "norm_ffn": e(L, d),
         "w_qkv": e(L, (Hq + 2 * Hkv) * D, d), "w_o": e(L, d, Hq * D), "w_gu": e(L, 2 * F, d),
         "w_down": e(L, d, F)}
    B.synth_xavier(W["embed"], synth.S_EMBED, d, V, seed)
    B.synth_xavier(W["lm_head"], synth.S_LMHEAD, d, V, seed)
    for k in ("norm_final", "norm_attn", "norm_ffn"):
        B.synth_fill(W[k], 1.0)
    for l in range(L):
        st = lambda t: synth.layer_stream(l, t)
        q0, k0, v0 = 0, Hq * D, (Hq + Hkv) * D
        B.synth_xavier(W["w_qkv"][l, q0:k0], st(synth.T_WQ), d, Hq * D, seed)
        B.synth_xavier(W["w_qkv"][l, k0:v0], st(synth.T_WK), d, Hkv * D, seed)
        B.synth_xavier(W["w_qkv"][l, v0:], st(synth.T_WV), d, Hkv * D, seed)
        B.synth_xavier(W["w_o"][l], st(synth.T_WO), Hq * D, d, seed)
        B.synth_xavier(W["w_gu"][l, :F], st(synth.T_W1), d, F, seed)
        B.synth_xavier(W["w_gu"][l, F:], st(synth.T_W3), d, F, seed)
        B.synth_xavier(W["w_down"][l], st(synth.T_W2), F, d, seed)
    return W


def compress_spec_desc(spec, shape, T: int, src_cap: int):
    dt = B.VC_BF16 if shape.dtype == "bf16" else B.VC_F32
    if spec.kind == "tokdrop" and spec.score == "keynorm":
        # the pages' example compressor: keep max(32, T // ratio) tokens, no recent window of its own
        return B.compress_desc(B.VC_TOKDROP, shape.n_layers, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, T, dt,
                               src_cap=src_cap, keep_total=max(32, T // spec.ratio), keep_recent=spec.keep_recent,
                               obs_window=0, score=B.VC_SCORE_KEYNORM)
    if spec.kind == "tokdrop":
        return B.compress_desc(B.VC_TOKDROP, shape.n_layers, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, T, dt,
                               src_cap=src_cap, keep_total=T // spec.ratio, keep_recent=spec.keep_recent,
                               obs_window=spec.obs_window)
    if spec.kind == "quant":
        return B.compress_desc(B.VC_QUANT, shape.n_layers, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, T, dt,
                               src_cap=src_cap, bits=spec.bits, group=spec.group)
    raise ValueError(spec.kind)


@dataclass
class Request:
    idx: int
    T: int
    x: int
    n_tokens: int
    cd: object = None
    comp: torch.Tensor = None
    tail_k: torch.Tensor = None
    tail_v: torch.Tensor = None
    full_k: object = None              # pinned host (HostBuffer)
    full_v: object = None
    n_host: int = 0                    # host rows per (layer, KV head)
    pinned: bool = True                # host rows in pinned memory (else pageable)
    stage_fut: object = None           # pageable staging in flight on the worker thread
    rows: torch.Tensor = None          # device int32 [x + 1]
    vtail_k: torch.Tensor = None
    vtail_v: torch.Tensor = None
    verified: torch.Tensor = None
    result: torch.Tensor = None
    result_host: torch.Tensor = None
    req: Req = None
    emitted: list = field(default_factory=list)
    accepts: list = field(default_factory=list)
    phase: int = DRAFT
    start_tick: int = 0
    slot: int = -1
    stage_ev: object = None
    acc_ev: object = None
    budget: int = -1                   # verifications it may still issue (-1: unlimited; 0: parked)
    x_cur: int = 0                     # this round's draft length (x unless adaptive; 0: a plain round)
    x_hist: list = field(default_factory=list)  # draft length of every verification issued
    zero_run: int = 0                  # consecutive rounds that kept no draft
    plain_left: int = 0                # plain rounds left before drafting is tried again
    n_verified: int = 0                # verifications issued
    rounds: list = field(default_factory=list)  # per-round record (Engine(record=True))
    rec_host: torch.Tensor = None      # pinned [2][x + 1]: this round's rows and verified tokens
    ready: object = None               # threading.Event: set once the compressed cache is on the device
                                       # (remote prefix shipping); None: it is there from the start
    t_first: float = None              # wall time at which the first round's tokens were known
    sampler: object = None             # _vc.Sampler (sampled decoding), else None (greedy)
    probs: torch.Tensor = None         # fp32 [x][vocab]: this round's draft distributions


class Engine:
    """Owns a vc_model, its workspaces and the per-request device/host buffers."""

    record = False
    temperature = None  # greedy unless a temperature is given

    # the driver pins at most ~70 GiB of host memory per process; rows beyond the budget
    # go to pageable memory, which no copy engine touches: they move one layer at a time
    # through a pinned pair of one-layer buffers (host memcpy on one side, a pinned copy on
    # the other), outside the budget and at most BOUNCE_MAX bytes
    PINNED_BUDGET = 69_000_000_000
    BOUNCE_MAX = 1_200_000_000

    def __init__(self, model: B.Model, spec, chunk: int = 1024, device="cuda", pinned_budget: int | None = None,
                 record: bool = False, temperature: float | None = None, seed: int = 0):
        """record: keep, per request and round, the position, the pending token, the drafts, the
        verifier's tokens and the accept count (host copies of device values; for parity tests).
        temperature: None decodes greedily (exact-match acceptance); a value >= 0 samples
        ("Mathematical Guarantee of Lossless Correctness", VeriCache Guide): drafts are drawn
        from the compressed cache's distribution and kept by speculative rejection sampling
        against the full-KV distribution, with the draws of request r taken from stream r of
        the generator keyed by seed."""
        self.m = model
        self.record = record
        self.temperature = temperature
        self.seed = seed
        self.vlogits = None
        self.ws_spec = None
        self.vargmax = None
        self.spec = spec
        self.shape = model.shape
        self.dt = torch.bfloat16 if self.shape.dtype == "bf16" else torch.float32
        self.chunk = chunk
        self.device = device
        self.reqs: list[Request] = []
        self.copy_stream = runtime.RT.Stream(device=device)
        self.slots = []
        self.slot_free_ev = []
        self.ws_draft = None
        self.ws_verify = None
        self.staged_bytes = 0          # host rows copied to the device for verification (both K and V)
        self.stagings = 0
        self.pinned_budget = self.PINNED_BUDGET if pinned_budget is None else pinned_budget
        self.pinned_used = 0
        self.pageable_stream = None
        self.stager = None
        self.bounce = None             # (K, V) pinned one-layer buffers for pageable host rows

    # ------------------------------------------------------------ setup (untimed)
    def add_request(self, prompt: torch.Tensor, x: int, n_tokens: int, keep_prefill_kv: bool = False):
        s = self.shape
        T = int(prompt.numel())
        L, Hkv, D, Hq = s.n_layers, s.n_kv_heads, s.head_dim, s.n_q_heads
        r = Request(idx=len(self.reqs), T=T, x=x, n_tokens=n_tokens)
        kd = torch.empty(L, Hkv, T, D, dtype=self.dt, device=self.device)
        vd = torch.empty_like(kd)
        W = min(self.spec.obs_window, T)
        q_obs = torch.empty(L, W, Hq, D, dtype=self.dt, device=self.device)
        g0 = torch.empty(1, dtype=torch.int32, device=self.device)
        ws = self.m.workspace(min(self.chunk, T), T, device=self.device)
        last = None
        if self.temperature is not None:
            r.sampler = B.Sampler(self.temperature, self.seed, r.idx)
            last = torch.empty(1, s.vocab, dtype=torch.float32, device=self.device)
            B.debug_register(last, g0)
        self.m.prefill(prompt, kd, vd, q_obs, W, g0, ws, min(self.chunk, T), last_logits=last)
        if last is not None:  # g0 drawn from the prompt's last row at position T
            B.vc_sample(last, [r.sampler], [T], B.VC_DRAW_TARGET, out=g0)
        if runtime.RT.dry:  # the first token the prefill would have written
            g0.fill_(1)
        del ws
        r.cd = compress_spec_desc(self.spec, s, T, T)
        r.comp = B.vc_compress(r.cd, kd, vd, q_obs)
        r.n_host = B.compress_layout(r.cd).n_host
        full_cap = max(r.n_host, 1)
        eb = 2 if self.dt == torch.bfloat16 else 4
        nbytes = L * Hkv * full_cap * D * eb
        r.pinned = self.pinned_used + 2 * nbytes <= self.pinned_budget
        if r.pinned:
            self.pinned_used += 2 * nbytes
        buf = B.HostBuffer if r.pinned else B.PageableBuffer
        r.full_k = buf(nbytes)
        r.full_v = buf(nbytes)
        if not r.pinned:
            self._bounce(nbytes // L)
        tail_cap = n_tokens + x + 2
        r.tail_k = torch.empty(L, Hkv, tail_cap, D, dtype=self.dt, device=self.device)
        r.tail_v = torch.empty_like(r.tail_k)
        r.rows = torch.zeros(x + 1, dtype=torch.int32, device=self.device)
        r.rows[:1].copy_(g0)
        r.vtail_k = torch.empty(L, Hkv, x + 1, D, dtype=self.dt, device=self.device)
        r.vtail_v = torch.empty_like(r.vtail_k)
        r.verified = torch.empty(x + 1, dtype=torch.int32, device=self.device)
        r.result = torch.empty(x + 2, dtype=torch.int32, device=self.device)
        r.result_host = torch.empty(x + 2, dtype=torch.int32, pin_memory=runtime.RT.pin)
        if self.record:
            r.rec_host = torch.empty(2, x + 1, dtype=torch.int32, pin_memory=runtime.RT.pin)
        if r.sampler is not None:
            r.probs = torch.empty(x, s.vocab, dtype=torch.float32, device=self.device)
            B.debug_register(r.probs)
        B.debug_register(r.rows, r.tail_k, r.tail_v, r.vtail_k, r.vtail_v, r.verified, r.result)
        r.req = Req(comp=r.comp.data_ptr(), cd=None, tail_k=r.tail_k.data_ptr(), tail_v=r.tail_v.data_ptr(),
                    tail_cap=tail_cap, n_tail=0, ctx_len=T, draft_idx=0,
                    full_k_host=r.full_k.data_ptr() if r.pinned else None,
                    full_v_host=r.full_v.data_ptr() if r.pinned else None, full_cap=full_cap,
                    rows=r.rows.data_ptr())
        import ctypes as C
        r.req.cd = C.pointer(r.cd)
        if r.pinned:
            self.m.offload(r.req, kd, vd, T)
        else:
            self._offload_pageable(r, kd, vd, T)
        runtime.RT.synchronize()
        r.emitted = [int(g0.item())]
        if r.emitted[0] < 0:
            raise NonFiniteLogits(f"request {r.idx}: the prefill's last row has no finite logit")
        if keep_prefill_kv:
            r.prefill_kv = (kd, vd)
            r.q_obs = q_obs
        self.reqs.append(r)
        return r

    def _alloc(self):
        s = self.shape
        n = len(self.reqs)
        max_ctx = max(r.T + r.n_tokens + r.x + 2 for r in self.reqs)
        max_x = max(r.x for r in self.reqs)
        self.ws_draft = self.m.workspace(min(n, 16), max_ctx, device=self.device)
        self.ws_verify = self.m.workspace(max_x + 1, max_ctx, device=self.device)
        if self.temperature is not None:
            self.vlogits = torch.empty(max_x + 1, s.vocab, dtype=torch.float32, device=self.device)
            self.ws_spec = torch.empty(B.spec_ws_size(max_x), dtype=torch.uint8, device=self.device)
            self.vargmax = torch.empty(max_x + 1, dtype=torch.int32, device=self.device)  # greedy picks, unused
            B.debug_register(self.vlogits, self.ws_spec, self.vargmax)
        L, Hkv, D = s.n_layers, s.n_kv_heads, s.head_dim
        n_slots = min(getattr(self, 'n_slots', 2), n)
        slot_rows = max(max(r.n_host for r in self.reqs), 1)
        if not self.slots:
            self.slots = [(torch.empty(L, Hkv, slot_rows, D, dtype=self.dt, device=self.device),
                           torch.empty(L, Hkv, slot_rows, D, dtype=self.dt, device=self.device))
                          for _ in range(n_slots)]
            self.slot_free_ev = [None] * n_slots
            self.slot_owner = [None] * n_slots

    # ------------------------------------------------------------ the VeriCache loop
    def start(self, lead: int | None = None, stagger: bool = True, draft_batch: int | None = None,
              queue_min: int = 1, n_slots: int = 3, adaptive: bool = False, x_min: int = 1,
              fallback_after: int = 0, plain_rounds: int = 8):
        """Allocate slots/workspaces and set the staggered start ticks.

        lead: a request's host rows start to stage once it has begun drafting and is within
        `lead` draft steps of its last draft.  None (default) stages as soon as drafting has
        begun: the sizing rule lead = ceil(t_copy / t_tick) gives more than x steps when one
        request's host rows take longer to copy than x draft steps take to run.
        draft_batch / queue_min: a request that has not begun its x drafts waits while at least
        queue_min drafted requests are queued for verification and fewer than draft_batch
        requests would draft together; drafting is then done in larger batches (fuller draft
        kernels) while the host link, which sets the pace, still always has a drafted request to
        stage.  draft_batch=1 drafts every request as soon as it can (default: all requests,
        counting only those not yet done).  A waiting request holds no slot, so the wait always
        ends: slot holders are drafting or drafted, and each verification returns a request to
        the waiting ones.
        n_slots: device staging buffers.  With fuller draft batches several requests finish
        drafting together; a third slot lets the link stage the next one while two staged
        requests wait for their verification.
        adaptive / x_min: per-request draft length ("Tuning and Scaling", VeriCache Guide: the
        drafting horizon is sized so that the full-KV copy overlaps drafting, L_min =
        ceil(t_copy / t_step); KV Cache and Speculative Decoding: a falling acceptance rate is the
        sign that speculation costs more than it saves).  A request starts at its x; after a
        round that accepts every draft its length doubles (at most x), after a rejection at a it
        becomes max(x_min, a + 1).  The emitted tokens do not change, only how many are drafted
        per verification.
        fallback_after / plain_rounds (adaptive only): after fallback_after consecutive rounds
        that keep no draft, the request decodes plainly for plain_rounds rounds (no drafts: each
        round verifies the pending token alone against the full KV and emits one token; "When
        the Serving Stack Breaks Down", KV Cache and Speculative Decoding), then drafts again at
        x_min.  0 never falls back."""
        self.n_slots = max(1, n_slots)
        self._alloc()
        n = len(self.reqs)
        for r in self.reqs:
            r.start_tick = (r.idx * r.x) // n if stagger else 0
            r.phase = DRAFT if len(r.emitted) < r.n_tokens else DONE
            r.budget = -1
            r.x_cur = r.x
        self.adaptive = adaptive
        self.x_min = max(1, x_min)
        self.fallback_after = fallback_after
        self.plain_rounds = plain_rounds
        for r in self.reqs:
            r.zero_run = r.plain_left = 0
        self.lead = max(r.x for r in self.reqs) if lead is None else lead
        self.draft_batch = n if draft_batch is None else max(1, draft_batch)
        self.queue_min = queue_min
        self.tick = 0
        self.draft_steps = 0
        self.drafted = 0  # request-tokens drafted (sum of the batch over draft steps)
        self.verifications = 0

    def step(self) -> bool:
        """One scheduler iteration: finish accepts, issue staging, one batched
        draft step, issue ready verifications.  Returns True if a draft step ran."""
        reqs = self.reqs
        cs = runtime.RT.current_stream()
        # 1. finish accepts whose result reached the host
        for r in reqs:
            if r.phase == ACCEPTING and r.acc_ev.query():
                self._finish_accept(r)
        # 2. stage full KV for requests close to the end of their draft (only once drafting has
        # begun: a request still waiting for a fuller draft batch must not hold a slot)
        for r in reqs:
            if (r.phase == DRAFT and r.slot < 0 and r.req.draft_idx >= max(1, r.x_cur - self.lead)
                    and self.tick >= r.start_tick and self._ready(r)):
                self._try_stage(r)
        # a request in a plain round (draft length 0) has nothing to draft
        for r in reqs:
            if r.phase == DRAFT and r.x_cur == 0 and r.budget != 0 and self.tick >= r.start_tick and self._ready(r):
                r.phase = WAIT_SLOT
        # 3. one batched draft step for every drafting request; requests yet to begin wait for a
        # fuller batch while enough drafted requests are queued for the host link
        ready = [r for r in reqs
                 if r.phase == DRAFT and r.budget != 0 and self.tick >= r.start_tick and r.req.draft_idx < r.x_cur
                 and self._ready(r)]
        active = [r for r in ready if r.req.draft_idx > 0]
        fresh = [r for r in ready if r.req.draft_idx == 0]
        queued = sum(1 for r in reqs if r.phase == WAIT_SLOT)
        # requests that will draft again (finished or parked ones never join a batch)
        live = sum(1 for r in reqs if r.phase != DONE and r.budget != 0)
        if fresh and (len(active) + len(fresh) >= min(self.draft_batch, live) or queued < self.queue_min):
            active += fresh
        for k in range(0, len(active), 16):
            grp = active[k:k + 16]
            if self.temperature is None:
                self.m.draft_step([r.req for r in grp], self.ws_draft)
            else:
                self.m.draft_step_sampled([r.req for r in grp], [r.sampler for r in grp], [r.probs for r in grp],
                                          self.ws_draft)
            self.drafted += len(grp)
            for r in grp:
                r.req.draft_idx += 1
                if r.req.draft_idx == r.x_cur:
                    r.phase = WAIT_SLOT
        # 4. verify requests whose drafts are complete and whose slot is staged
        for r in reqs:
            if r.phase == WAIT_SLOT:
                if r.slot < 0:
                    self._try_stage(r)
                if r.slot >= 0 and self._staged(r):
                    self._verify(r, cs)
        if active:
            self.draft_steps += 1
        self.tick += 1
        return bool(active)

    @staticmethod
    def _ready(r: Request) -> bool:
        return r.ready is None or r.ready.is_set()

    def _finish_accept(self, r: Request):
        a = int(r.result_host[0])
        if r.t_first is None:
            r.t_first = time.perf_counter()
        if self.record:
            n = r.x_cur + 1
            rows, ver = r.rec_host[0, :n].tolist(), r.rec_host[1, :n].tolist()
            if self.temperature is not None:  # the verifier's tokens after a are not written
                ver = ver[:a + 1]
            r.rounds.append({"pos": r.req.ctx_len, "n_tail": r.req.n_tail, "pending": rows[0], "draft": rows[1:],
                             "verified": ver, "a": a})
        new = r.result_host[1:a + 2].tolist()
        if min(new) < 0:
            raise NonFiniteLogits(f"request {r.idx}: a row of its round {len(r.accepts)} (position "
                                  f"{r.req.ctx_len} onwards) has no finite logit; emitted {new}")
        r.emitted += new
        r.accepts.append(a)
        if self.adaptive:
            self._next_x(r, a)
        self.m.commit(r.req, a, r.vtail_k, r.vtail_v, after_event=r.acc_ev, copy_stream=self.copy_stream)
        r.phase = DRAFT if len(r.emitted) < r.n_tokens else DONE

    def _next_x(self, r: Request, a: int):
        """The next round's draft length after a round that kept a drafts (see start)."""
        if r.x_cur == 0:
            r.plain_left -= 1
            if r.plain_left <= 0:
                r.x_cur, r.zero_run = min(self.x_min, r.x), 0
            return
        r.zero_run = r.zero_run + 1 if a == 0 else 0
        if self.fallback_after and r.zero_run >= self.fallback_after:
            r.x_cur, r.plain_left = 0, self.plain_rounds
        elif a == r.x_cur:
            r.x_cur = min(r.x, 2 * r.x_cur)
        else:
            r.x_cur = max(min(self.x_min, r.x), a + 1)

    def drain(self):
        """Wait for every in-flight verification and fold its accepted tokens in."""
        runtime.RT.synchronize()
        for r in self.reqs:
            if r.phase == ACCEPTING:
                r.acc_ev.synchronize()
                self._finish_accept(r)
        self.copy_stream.synchronize()

    def emitted_total(self) -> int:
        return sum(len(r.emitted) for r in self.reqs)

    def run(self, lead: int | None = None, stagger: bool = True, trace: list | None = None, adaptive: bool = False,
            x_min: int = 1, fallback_after: int = 0, plain_rounds: int = 8):
        """Decode every request to its n_tokens; returns wall seconds of the decode phase."""
        self.start(lead, stagger, adaptive=adaptive, x_min=x_min, fallback_after=fallback_after,
                   plain_rounds=plain_rounds)
        t0 = time.perf_counter()
        while any(r.phase != DONE for r in self.reqs):
            self.step()
            if trace is not None:
                trace.append((self.tick, [r.phase for r in self.reqs], [r.req.draft_idx for r in self.reqs]))
        self.drain()
        for r in self.reqs:
            r.emitted = r.emitted[: r.n_tokens]
        return time.perf_counter() - t0

    def run_draft_steps(self, n: int):
        """Run scheduler iterations until n more batched draft steps have executed."""
        target = self.draft_steps + n
        while self.draft_steps < target and any(r.phase != DONE for r in self.reqs):
            self.step()

    def run_rounds(self, n: int):
        """Run scheduler iterations until n more verifications have been issued (a fixed
        amount of decoding work whatever the draft batching; drain() completes them)."""
        target = self.verifications + n
        while self.verifications < target and any(r.phase != DONE for r in self.reqs):
            self.step()

    def run_rounds_each(self, n: int):
        """Let every unfinished request issue exactly n more verifications (a request that has
        issued them parks: it neither drafts nor stages); returns once all are issued, and
        drain() completes them.  Drafts and verifications do not depend on which requests
        share a draft step, so the tokens these rounds emit do not depend on the schedule."""
        for r in self.reqs:
            r.budget = n if r.phase != DONE else 0
        while any(r.phase != DONE and r.budget > 0 for r in self.reqs):
            self.step()

    def run_to_end(self, progress=None, every: float = 20.0):
        """Lift every request's round budget and decode until all have their token count;
        progress(emitted tokens, seconds) is called about every `every` seconds."""
        for r in self.reqs:
            if r.phase != DONE:
                r.budget = -1
        t0 = t_last = time.perf_counter()
        while any(r.phase != DONE for r in self.reqs):
            if not self.step() and any(not self._ready(r) for r in self.reqs):
                time.sleep(0.0005)  # waiting on a cache in flight: leave the interpreter to the link's thread
            if progress is not None and time.perf_counter() - t_last >= every:
                t_last = time.perf_counter()
                progress(sum(min(len(r.emitted), r.n_tokens) for r in self.reqs), t_last - t0)
        self.drain()

    def _try_stage(self, r: Request):
        for i in range(len(self.slots)):
            if self.slot_owner[i] is None and (self.slot_free_ev[i] is None or self.slot_free_ev[i].query()):
                self.slot_owner[i] = r.idx
                r.slot = i
                sk, sv = self.slots[i]
                self.staged_bytes += 2 * sk[:, :, :r.n_host].numel() * sk.element_size()
                self.stagings += 1
                if r.pinned:
                    self.m.stage(r.req, sk, sv, 0, self.shape.n_layers, copy_stream=self.copy_stream)
                    ev = runtime.RT.Event()
                    ev.record(self.copy_stream)
                    r.stage_ev = ev
                else:
                    r.stage_ev = None
                    r.stage_fut = self._stage_pageable(r, sk, sv)
                return True
        return False

    # ------------------------------------------------------------ pageable host rows
    def _bounce(self, layer_bytes: int):
        """The pinned (K, V) pair of one-layer buffers, grown to layer_bytes if needed."""
        if self.bounce is not None and self.bounce[0].nbytes >= layer_bytes:
            return self.bounce
        if 2 * layer_bytes > self.BOUNCE_MAX:
            raise ValueError(f"a layer of host rows ({layer_bytes} B) exceeds the pinned staging pair")
        if self.bounce is not None:
            runtime.RT.synchronize()
            if self.pageable_stream is not None:
                self.pageable_stream.synchronize()
            for b in self.bounce:
                b.free()
        self.bounce = (B.HostBuffer(layer_bytes), B.HostBuffer(layer_bytes))
        return self.bounce

    @staticmethod
    def _layer_req(r: Request, bk, bv, l: int, lb: int) -> Req:
        """r's request with host arrays placed so that layer l lies in the pinned pair (the
        library touches only the layers it is given)."""
        q = Req.from_buffer_copy(r.req)
        q.full_k_host = bk.data_ptr() - l * lb
        q.full_v_host = bv.data_ptr() - l * lb
        return q

    def _offload_pageable(self, r: Request, kd, vd, T: int):
        """Offload into pageable memory one layer at a time: the library copies layer l into
        the pinned pair, the host copies it on into the pageable store."""
        L = self.shape.n_layers
        lb = r.full_k.nbytes // L
        bk, bv = self.bounce
        for l in range(L):
            self.m.offload(self._layer_req(r, bk, bv, l, lb), kd, vd, T, l, l + 1)
            runtime.RT.synchronize()
            if not runtime.RT.dry:
                r.full_k.t[l * lb:(l + 1) * lb].copy_(bk.tensor()[:lb])
                r.full_v.t[l * lb:(l + 1) * lb].copy_(bv.tensor()[:lb])

    def _stage_pageable(self, r: Request, sk, sv):
        """Stage from pageable memory on a worker thread: per layer, a host copy into the
        pinned pair, then the library's pinned copy into the slot; the pair is reused once
        that copy has completed."""
        if self.stager is None:
            self.stager = cf.ThreadPoolExecutor(max_workers=1)
            self.pageable_stream = runtime.RT.Stream(device=self.device)
        st = self.pageable_stream
        L = self.shape.n_layers
        lb = r.full_k.nbytes // L
        bk, bv = self.bounce

        def work():
            ev = runtime.RT.Event()
            for l in range(L):
                if not runtime.RT.dry:
                    bk.tensor()[:lb].copy_(r.full_k.t[l * lb:(l + 1) * lb])
                    bv.tensor()[:lb].copy_(r.full_v.t[l * lb:(l + 1) * lb])
                self.m.stage(self._layer_req(r, bk, bv, l, lb), sk, sv, l, l + 1, copy_stream=st)
                ev = runtime.RT.Event()
                ev.record(st)
                ev.synchronize()
            return ev

        return self.stager.submit(work)

    def _staged(self, r: Request) -> bool:
        if r.stage_ev is None and r.stage_fut is not None and r.stage_fut.done():
            r.stage_ev = r.stage_fut.result()
            r.stage_fut = None
        return r.stage_ev is not None and r.stage_ev.query()

    def release_host(self):
        """Free every request's host buffers (after decoding)."""
        if self.stager is not None:
            self.stager.shutdown(wait=True)
            self.stager = None
        if self.pageable_stream is not None:
            self.pageable_stream.synchronize()
        for r in self.reqs:
            for b in (r.full_k, r.full_v):
                if b is not None:
                    b.free()
            r.full_k = r.full_v = None
        if self.bounce is not None:
            for b in self.bounce:
                b.free()
            self.bounce = None
        self.pinned_used = 0

    def _verify(self, r: Request, cs):
        self.verifications += 1
        r.x_hist.append(r.x_cur)
        if r.budget > 0:
            r.budget -= 1
        sk, sv = self.slots[r.slot]
        if self.temperature is None:
            self.m.verify(r.req, sk, sv, r.rows, r.x_cur + 1, r.verified, r.vtail_k, r.vtail_v, self.ws_verify)
        else:  # the verify rows' logits, then rejection sampling writes the tokens vc_accept compares
            self.m.verify(r.req, sk, sv, r.rows, r.x_cur + 1, self.vargmax, r.vtail_k, r.vtail_v, self.ws_verify,
                          logits=self.vlogits)
            B.vc_spec_sample(self.vlogits[:r.x_cur + 1], r.probs, r.rows.data_ptr() + 4, r.x_cur, r.sampler,
                             r.req.ctx_len, r.verified, self.ws_spec)
        if self.record:  # before vc_accept overwrites rows[0] with the next pending token
            n = r.x_cur + 1
            r.rec_host[0, :n].copy_(r.rows[:n], non_blocking=True)
            r.rec_host[1, :n].copy_(r.verified[:n], non_blocking=True)
        ev_free = runtime.RT.Event()
        ev_free.record(cs)
        self.slot_free_ev[r.slot] = ev_free
        self.slot_owner[r.slot] = None
        r.slot = -1
        self.m.accept(r.req, r.verified, r.x_cur, r.vtail_k, r.vtail_v, r.result)
        if runtime.RT.dry:  # the accept result the library would have written
            runtime.RT.fill_accept(r.idx, r.n_verified, r.x_cur, r.result)
        r.n_verified += 1
        r.result_host.copy_(r.result, non_blocking=True)
        ev = runtime.RT.Event()
        ev.record(cs)
        r.acc_ev = ev
        r.phase = ACCEPTING


# ---------------------------------------------------------------- greedy baselines
def greedy_resident(model: B.Model, prompt: torch.Tensor, n_tokens: int, chunk: int = 1024, device="cuda"):
    """Full-KV greedy decoding with the cache resident in HBM: each step is
    vc_verify with one row, writing its K/V straight into the cache."""
    s = model.shape
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    T = int(prompt.numel())
    cap = T + n_tokens
    L, Hkv, D = s.n_layers, s.n_kv_heads, s.head_dim
    kd = torch.empty(L, Hkv, cap, D, dtype=dt, device=device)
    vd = torch.empty_like(kd)
    out = (torch.ones if runtime.RT.dry else torch.empty)(n_tokens, dtype=torch.int32, device=device)
    ws = model.workspace(min(chunk, T), cap, device=device)
    B.debug_register(kd, vd, out, ws)
    model.prefill(prompt, kd, vd, None, 0, out[:1], ws, min(chunk, T))
    req = Req(ctx_len=T)
    eb = 2 if s.dtype == "bf16" else 4
    row = D * eb
    t0 = None
    runtime.RT.synchronize()
    t0 = time.perf_counter()
    for i in range(1, n_tokens):
        req.ctx_len = T + i - 1
        off = req.ctx_len * row
        model.verify_raw(req, kd.data_ptr(), vd.data_ptr(), cap, out.data_ptr() + 4 * (i - 1), 1,
                         out.data_ptr() + 4 * i, kd.data_ptr() + off, vd.data_ptr() + off, cap, ws)
    runtime.RT.synchronize()
    toks = out.tolist()
    if min(toks) < 0:
        raise NonFiniteLogits(f"greedy decoding: token -1 at step {toks.index(-1)}")
    return toks, time.perf_counter() - t0, (kd, vd)


def sample_resident(model: B.Model, prompt: torch.Tensor, n_tokens: int, sampler, chunk: int = 1024, device="cuda"):
    """Full-KV sampled decoding with the cache resident in HBM (the distribution sampled
    VeriCache must reproduce): the token at position p is drawn from the row before it with
    the TARGET draw of p (g0 from the prompt's last row at position T)."""
    s = model.shape
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    T = int(prompt.numel())
    cap = T + n_tokens
    L, Hkv, D = s.n_layers, s.n_kv_heads, s.head_dim
    kd = torch.empty(L, Hkv, cap, D, dtype=dt, device=device)
    vd = torch.empty_like(kd)
    out = torch.empty(n_tokens, dtype=torch.int32, device=device)
    logits = torch.empty(1, s.vocab, dtype=torch.float32, device=device)
    pick = torch.empty(1, dtype=torch.int32, device=device)
    ws = model.workspace(min(chunk, T), cap, device=device)
    B.debug_register(kd, vd, out, logits, pick, ws)
    model.prefill(prompt, kd, vd, None, 0, pick, ws, min(chunk, T), last_logits=logits)
    B.vc_sample(logits, [sampler], [T], B.VC_DRAW_TARGET, out=out[:1])
    req = Req(ctx_len=T)
    row = D * (2 if s.dtype == "bf16" else 4)
    for i in range(1, n_tokens):
        req.ctx_len = T + i - 1
        off = req.ctx_len * row
        model.verify_raw(req, kd.data_ptr(), vd.data_ptr(), cap, out.data_ptr() + 4 * (i - 1), 1, pick.data_ptr(),
                         kd.data_ptr() + off, vd.data_ptr() + off, cap, ws, logits=logits.data_ptr())
        B.vc_sample(logits, [sampler], [T + i], B.VC_DRAW_TARGET, out=out[i:i + 1])
    runtime.RT.synchronize()
    toks = out.tolist()
    if min(toks) < 0:
        raise NonFiniteLogits(f"sampled decoding: token -1 at step {toks.index(-1)}")
    return toks


def greedy_from_host(model: B.Model, prompt_kv, T: int, first_token: torch.Tensor, n_steps: int, ws: torch.Tensor,
                     copy_stream, layered: bool = True):
    """Full-KV greedy decoding with the cache in pinned host memory, the
    comparator VeriCache is measured against: a plain request (no compressed
    cache) whose whole context lives on the host; every token stages it over
    PCIe, runs one verification row, and appends the new row to the host copy.
    layered: the context is staged one layer at a time and layer l's attention
    waits only for layer l (vc_verify_layered), so each layer's compute overlaps
    the copies of the layers after it; otherwise all layers are staged before
    vc_verify starts.
    prompt_kv: device (K, V) [L][Hkv][cap][D] holding prompt rows [0, T);
    first_token: device int32 [1], the token at position T.
    Returns (tokens after first_token, seconds)."""
    s = model.shape
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    L, Hkv, D = s.n_layers, s.n_kv_heads, s.head_dim
    eb = 2 if dt == torch.bfloat16 else 4
    cap = T + n_steps + 1
    hk = B.HostBuffer(L * Hkv * cap * D * eb)
    hv = B.HostBuffer(L * Hkv * cap * D * eb)
    sk = torch.empty(L, Hkv, cap, D, dtype=dt, device=prompt_kv[0].device)
    sv = torch.empty_like(sk)
    vk = torch.empty(L, Hkv, 1, D, dtype=dt, device=sk.device)
    vv = torch.empty_like(vk)
    rows = first_token.clone()
    B.debug_register(sk, sv, vk, vv, rows, ws)
    req = Req(ctx_len=T, full_k_host=hk.data_ptr(), full_v_host=hv.data_ptr(), full_cap=cap, rows=rows.data_ptr())
    model.offload(req, prompt_kv[0], prompt_kv[1], T)
    cs = runtime.RT.current_stream()
    toks = []
    runtime.RT.synchronize()
    t0 = time.perf_counter()
    layer_ev = [runtime.RT.Event() for _ in range(L)]
    committed = None
    for _ in range(n_steps):
        if layered:
            for l in range(L):
                model.stage(req, sk, sv, l, l + 1, copy_stream=copy_stream)
                layer_ev[l].record(copy_stream)
            # the verification writes its new rows into vk / vv in each layer's projections,
            # before that layer waits for its staged rows: it must not start while the previous
            # step's commit still copies them out
            if committed is not None:
                cs.wait_event(committed)
            model.verify_layered_raw(req, sk.data_ptr(), sv.data_ptr(), cap, rows.data_ptr(), 1, rows.data_ptr(),
                                     vk.data_ptr(), vv.data_ptr(), 1, ws, layer_ev)
        else:
            model.stage(req, sk, sv, 0, L, copy_stream=copy_stream)
            ev = runtime.RT.Event()
            ev.record(copy_stream)
            cs.wait_event(ev)
            model.verify_raw(req, sk.data_ptr(), sv.data_ptr(), cap, rows.data_ptr(), 1, rows.data_ptr(),
                             vk.data_ptr(), vv.data_ptr(), 1, ws)
        done = runtime.RT.Event()
        done.record(cs)
        model.commit(req, 0, vk, vv, after_event=done, copy_stream=copy_stream)
        committed = runtime.RT.Event()
        committed.record(copy_stream)
        toks.append(rows.clone())
    runtime.RT.synchronize()
    copy_stream.synchronize()
    secs = time.perf_counter() - t0
    del sk, sv
    hk.free()
    hv.free()
    toks = [int(t.item()) for t in toks]
    if toks and min(toks) < 0:
        raise NonFiniteLogits(f"full-KV-from-host decoding: token -1 at step {toks.index(-1)}")
    return toks, secs
