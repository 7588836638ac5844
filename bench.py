#!/usr/bin/env python3
"""Lossless decode throughput of the VeriCache draft/verify loop on one MI355X.

Default workload: the 32-layer Llama-3-8B-shaped random-init decoder (bf16),
8 requests with 65536-token prompts, a 4x token-dropped draft cache on the GPU,
the rest of the full KV cache (the dropped prompt rows; the kept rows and the
committed tail are exact on the GPU) in pinned host memory, staged over PCIe
only to verify, x = 32, staggered verification.  A step is one verification round per
request: in the timed region every request issues its verification rounds warmup + 1 ..
warmup + steps (fewer if it reaches the workload's token count first; a request that is
done with them waits), and the region ends when they have completed: the same decoding
work, and the same emitted tokens, whatever the draft batching.

Reported: emitted (lossless) tokens per second over exactly --steps steps,
the live HIP-event time and algorithmic bytes of the draft-attention kernels
in the timed region (roofline vs 8 TB/s HBM), the full-KV-from-host greedy
comparator measured on the same requests, and the CPU oracle's rate on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
PCIE_PEAK_GBS = 63.0
# prompt rows per prefill chunk: 8192 rows give every 8B projection a whole number of rounds of
# 256 x 256 GEMM tiles over the 256 compute units (2048 rows leave half the GPU idle on 4096 columns)
PREFILL_CHUNK = 8192
PCIE_PINNED_GBS = 57.6  # pinned host-to-device rate measured on the box (4 GiB copy)  # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 / 8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(shape, ctx: int, keep: int, seed: int = 0) -> dict:
    """The oracle, as written, on a bounded sample of the workload: one layer of
    one draft step of request 0 (the layer's weights from the seeded recipe,
    attention over `keep` kept rows per KV head), repeated, plus the LM head on
    1/8 of the vocabulary; scaled to tokens/s of one drafting request."""
    import numpy as np
    import threadpoolctl

    import synth
    from oracle.model import attend, rmsnorm, rope, silu
    from oracle.rounding import to_bf16 as R
    s = shape
    D, Hq, Hkv, G = s.head_dim, s.n_q_heads, s.n_kv_heads, s.group
    st = lambda t: synth.layer_stream(0, t)
    mat = lambda stream, o, i: synth.bf16_bits_to_f32(synth.gen_bf16(synth.xavier(stream, (o, i), i, o, seed))).astype(np.float64)
    t_gen = time.perf_counter()
    Wq, Wk, Wv = mat(st(synth.T_WQ), Hq * D, s.d_model), mat(st(synth.T_WK), Hkv * D, s.d_model), mat(st(synth.T_WV), Hkv * D, s.d_model)
    Wo = mat(st(synth.T_WO), s.d_model, Hq * D)
    W1, W3, W2 = mat(st(synth.T_W1), s.ffn, s.d_model), mat(st(synth.T_W3), s.ffn, s.d_model), mat(st(synth.T_W2), s.d_model, s.ffn)
    v_slice = s.vocab // 8
    Wlm = mat(synth.S_LMHEAD, v_slice, s.d_model)
    Kc = [synth.bf16_bits_to_f32(synth.att_head(synth.S_ATT_K, 0, j, keep, Hkv, D)).astype(np.float64) for j in range(Hkv)]
    Vc = [synth.bf16_bits_to_f32(synth.att_head(synth.S_ATT_V, 0, j, keep, Hkv, D)).astype(np.float64) for j in range(Hkv)]
    t_gen = time.perf_counter() - t_gen
    h = R(np.ones(s.d_model) * 0.01)
    g = np.ones(s.d_model)
    reps = 2

    def layer(h):
        a = R(rmsnorm(h, g, s.eps))
        q = R(rope((Wq @ a).reshape(Hq, D), ctx, s.rope_theta))
        k = R(rope((Wk @ a).reshape(Hkv, D), ctx, s.rope_theta))
        v = R((Wv @ a).reshape(Hkv, D))
        o = np.stack([attend(q[hh], np.concatenate([Kc[hh // G], k[hh // G][None]]),
                             np.concatenate([Vc[hh // G], v[hh // G][None]])) for hh in range(Hq)])
        h = R(h + Wo @ R(o).reshape(-1))
        f = R(rmsnorm(h, g, s.eps))
        return R(h + W2 @ R(silu(W1 @ f) * (W3 @ f)))

    with threadpoolctl.threadpool_limits(None) as _:
        info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    t0 = time.perf_counter()
    for _ in range(reps):
        h = layer(h)
    t_layer = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    _ = Wlm @ R(rmsnorm(h, g, s.eps))
    t_lm = (time.perf_counter() - t0) * 8
    per_token = s.n_layers * t_layer + t_lm
    return {"value": 1.0 / per_token, "unit": "draft tokens/s (one request)", "cores": threads, "kind": "oracle",
            "sample": (f"{reps} evaluations of layer 0 of one draft step (attention over {keep} kept rows per KV "
                       f"head at position {ctx}) + LM head on 1/8 of the vocabulary, scaled to "
                       f"{s.n_layers} layers; {per_token:.2f} s per token; weight generation {t_gen:.1f} s excluded"),
            "host": host_info(), "tiny_workload_full_run": cpu_oracle_tiny()}


def host_info() -> dict:
    """The host the oracle ran on: cores, affinity, the BLAS library behind numpy and its threads."""
    import numpy  # noqa: F401  (loads the BLAS library threadpoolctl reports)
    import threadpoolctl
    info = threadpoolctl.threadpool_info()
    blas = [{"api": i.get("internal_api"), "version": i.get("version"), "threads": i.get("num_threads")}
            for i in info if i.get("user_api") == "blas"]
    return {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "blas": blas}


def cpu_oracle_tiny() -> dict:
    """The oracle's whole run of the tiny fp32 decoder workload (1024-token prompt, token drop 4x,
    x = 8, 64 tokens): prefill, full-KV greedy decoding and the VeriCache loop, all threads and one
    thread; tokens/s of each decode (the first token from the prefill excluded)."""
    import threadpoolctl

    import synth
    from oracle import decode as OD
    from oracle.model import Weights
    from synth.configs import tiny
    w = tiny()
    s = w.model
    W = Weights(s)
    p = synth.prompt(0, w.ctx[0], s.vocab)
    out = {}
    for label, limit in (("all_threads", None), ("one_thread", 1)):
        with threadpoolctl.threadpool_limits(limit):
            t0 = time.perf_counter()
            pre = OD.prefill(W, p)
            t1 = time.perf_counter()
            g, _ = OD.greedy(W, p, w.n_tokens, pre=pre)
            t2 = time.perf_counter()
            v, rounds = OD.vericache(W, p, w.n_tokens, w.x[0],
                                     lambda pr: OD.draft_cache_tokdrop(pr, W, keep_total=w.ctx[0] // 4, keep_recent=64),
                                     pre=pre)
            t3 = time.perf_counter()
        assert v == g, "oracle VeriCache differs from oracle greedy"
        out[label] = {"prefill_s": round(t1 - t0, 3), "greedy_tok_s": round((w.n_tokens - 1) / (t2 - t1), 2),
                      "vericache_tok_s": round((w.n_tokens - 1) / (t3 - t2), 2), "rounds": len(rounds)}
    return out


def pmc_traffic_ratio(workload: str, kernel: str = "attn_decode_bf16", what: str = "draft_attention"):
    """Measured HBM bytes over algorithmic bytes of one kernel class's launches, from the
    committed counter profile of this workload (profiles/<what>_<workload>_pmc.json),
    if the kernel sources are unchanged since.  The
    counter passes serialise every dispatch, which changes how many requests draft together,
    so the ratio (taken over the same launches on both sides) carries over to this run's
    launches rather than the profiled run's bytes per launch."""
    from lossless_speculative_decoding_amd.pmc_summary import sources_sha256
    path = os.path.join(ROOT, "profiles", f"{what}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel") != kernel or rec.get("sources_sha256") != sources_sha256(kernel):
        log(f"{path}: kernel sources changed since the counters were taken; traffic not reported")
        return None
    return rec.get("traffic_over_algorithmic")


def cpu_baseline_layer(T: int, Hq: int, Hkv: int, D: int, rows: int, bits: int, group: int) -> dict:
    """The oracle, as written, on one (request, KV head) slice of the single-layer workload:
    the draft step's attention over the dequantized cache for the G query heads, and the
    verification attention of all rows; reported as algorithmic bytes of that slice / time."""
    import threadpoolctl

    from oracle import attention as OA
    from oracle import compress as OC
    from oracle.model import attend
    import numpy as np
    inp = OA.head_inputs(0, 0, T, Hkv, Hq, D, rows)
    q = OC.Quantized(inp["K"][None, None], inp["V"][None, None], bits, group)   # compression: not timed
    with threadpoolctl.threadpool_limits(None) as _:
        info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    times = {}
    for label, limit in (("all", None), ("one", 1)):
        with threadpoolctl.threadpool_limits(limit):
            t0 = time.perf_counter()
            K = np.concatenate([q.rows_K()[0, 0], inp["tK"][:1]])
            V = np.concatenate([q.rows_V()[0, 0], inp["tV"][:1]])
            _ = [attend(qh, K, V) for qh in inp["qd"]]
            t_draft = time.perf_counter() - t0
            t0 = time.perf_counter()
            _ = OA.verify_output(inp)
            t_verify = time.perf_counter() - t0
        times[label] = (t_draft, t_verify)
    t_draft, t_verify = times["all"]
    Tq = T // group * group
    draft_bytes = 2 * Tq * D * bits / 8 + 2 * (Tq // group) * D * 2 + 2 * Tq * (D // group) * 2 + 2 * D * 2 \
        + (Hq // Hkv) * D * 2
    verify_bytes = 2 * (T + rows) * D * 2 + rows * (Hq // Hkv) * D * 2
    return {"value": round(draft_bytes / t_draft / 1e9, 4), "unit": "GB/s (draft attention, algorithmic bytes)",
            "cores": threads, "kind": "oracle",
            "verify_gbs": round(verify_bytes / t_verify / 1e9, 4),
            "one_thread": {"draft_gbs": round(draft_bytes / times["one"][0] / 1e9, 4),
                           "verify_gbs": round(verify_bytes / times["one"][1] / 1e9, 4)},
            "host": host_info(),
            "sample": (f"request 0, KV head 0 of the workload: draft attention of its {Hq // Hkv} query heads over "
                       f"the dequantized {T}-row cache ({t_draft:.2f} s) and verification attention of {rows} rows "
                       f"({t_verify:.2f} s), float64 numpy; quantization excluded")}


def bench_layer(args):
    """Single GQA attention layer (Llama-3-8B head shapes): a step is one batched draft-step
    attention of every request over its quantized cache plus one batched verification attention
    of its rows over the full bf16 cache."""
    import numpy as np
    import torch

    import synth
    from synth import configs
    import lossless_speculative_decoding_amd as vc
    from lossless_speculative_decoding_amd._vc import AttnDesc
    w = configs.gqa_layer()
    e = w.extra
    Hq, Hkv, D, rows = e["n_q_heads"], e["n_kv_heads"], e["head_dim"], e["verify_rows"]
    B, T, bits, group = w.batch, w.ctx[0], w.compress.bits, w.compress.group
    # other cache shapes of the same layer (the quantized caches of the 8B-shaped workloads: 2-bit
    # group 64 at 4 x 131072, 3-bit group 128 at 16 requests); the workload name records them
    B, T = args.batch or B, args.ctx or T
    bits, group = args.bits or bits, args.group or group
    name = w.name if (B, T, bits, group) == (w.batch, w.ctx[0], w.compress.bits, w.compress.group) else \
        f"gqa_layer_bf16_b{B}_t{T}_q{bits}g{group}"
    torch.cuda.set_device(0)

    def gen(shape, stream, outl=None, scale=1.0):
        t = torch.empty(*shape, dtype=torch.bfloat16, device="cuda")
        vc.synth_normal_heads(t, stream, outl, scale)
        return t

    outl = torch.from_numpy(np.stack([synth.outlier_channels_for(b, j, Hkv, D) for b in range(B)
                                      for j in range(Hkv)]).astype(np.int32)).cuda()
    K = gen((B, Hkv, T, D), synth.S_ATT_K, outl, e["outlier_scale"])
    V = gen((B, Hkv, T, D), synth.S_ATT_V, outl, e["outlier_scale"])
    tK = gen((B, Hkv, rows, D), synth.S_ATT_TK)
    tV = gen((B, Hkv, rows, D), synth.S_ATT_TV)
    qd = gen((1, B, Hq, D), synth.S_ATT_QD)[0]
    qv = gen((1, B * rows, Hq, D), synth.S_ATT_QV)[0].view(B, rows, Hq, D)
    cds, blobs = [], []
    for b in range(B):
        d = vc.compress_desc(vc.VC_QUANT, 1, Hq, Hkv, D, T, vc.VC_BF16, bits=bits, group=group)
        cds.append(d)
        blobs.append(vc.vc_compress(d, K[b:b + 1], V[b:b + 1]))
    torch.cuda.synchronize()
    desc = AttnDesc(Hq, Hkv, D, vc.VC_BF16, 0, vc.VC_BF16)
    Ks, Vs = [K[b] for b in range(B)], [V[b] for b in range(B)]
    tKs, tVs = [tK[b] for b in range(B)], [tV[b] for b in range(B)]

    def step():
        vc.vc_attn_draft(desc, blobs, cds, tKs, tVs, [1] * B, qd)
        vc.vc_attn_verify(desc, qv, Ks, Vs, [T] * B, tKs, tVs, rows)

    kinds = (vc.VC_PROF_DRAFT_ATTN, vc.VC_PROF_VERIFY_ATTN)
    vc.profile_enable(kinds)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    for k in kinds:
        vc.profile_read(k)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    secs = time.perf_counter() - t0
    vc.profile_enable(())
    dp, vp = vc.profile_read(vc.VC_PROF_DRAFT_ATTN), vc.profile_read(vc.VC_PROF_VERIFY_ATTN)
    dr = _rate(dp, "hbm", f"quantized draft attention partials, {B} requests x {Hkv} KV heads x {T} keys, "
                          f"{bits}-bit group {group}")
    vr = _rate(vp, "hbm", f"verification attention partials, {B} requests x {rows} rows x {Hq} heads over "
                          f"{T} + {rows} keys")
    ratio = pmc_traffic_ratio(name, "attn_quant")
    dr["traffic"] = round(ratio * dr["bytes_per_launch"]) if ratio else None
    dr["traffic_over_algorithmic"] = ratio
    ratio = pmc_traffic_ratio(f"{name[:name.rindex('_')]}_r{rows}", "attn_rows_bf16", "verify_attention")
    vr["traffic"] = round(ratio * vr["bytes_per_launch"]) if ratio else None
    vr["traffic_over_algorithmic"] = ratio
    cpu = None if args.no_cpu_baseline else cpu_baseline_layer(T, Hq, Hkv, D, rows, bits, group)
    line = {
        "metric": "draft-attn HBM GB/s vs peak (single GQA layer)",
        "value": dr["achieved"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(1000 * secs / args.steps, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) K/V with 4 outlier channels x10)",
        "config": {"workload": name, "batch": B, "ctx": T, "bits": bits, "group": group, "verify_rows": rows},
        "roofline": dr, "verify_attention": vr, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _rate(st: dict, bound: str, what: str) -> dict | None:
    """Live-timed kernel class against its roof: HBM bytes/s or bf16 MFMA flop/s."""
    if not st or st["launches"] == 0 or st["ms"] <= 0:
        return None
    secs = st["ms"] * 1e-3
    gbs = st["bytes"] / secs / 1e9
    tflops = st["flops"] / secs / 1e12
    if bound == "hbm":
        out = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(gbs / HBM_PEAK_GBS, 4), "tflops": round(tflops, 2)}
    else:
        out = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
               "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "gbs": round(gbs, 1)}
    out.update({"kernel": what, "launches": st["launches"], "avg_launch_ms": round(st["ms"] / st["launches"], 5),
                "bytes_per_launch": round(st["bytes"] / st["launches"]),
                "partial_bytes_per_launch": round(st.get("aux_bytes", 0) / st["launches"]),
                "flops_per_launch": round(st["flops"] / st["launches"])})
    return out


# Workloads refused by bench.py until the cause of a failure is shown.
DISABLED = {
    "llama8b_mixed": "its one run faulted the GPU although every launch and copy was range-checked first; the cause "
                     "found since (host rows beyond the pinned budget handed to the copy engines in pageable "
                     "memory) is fixed (they now move through a pinned pair of one-layer buffers), but the "
                     "workload has not run again yet",
}


def run_model_workload(args) -> dict:
    """The model workloads: setup (weights, prefill, compression, offload of every request),
    warmup and timed verification rounds, the compressed-only and comparator passes.  Runs on
    the selected runtime: the GPU, or a dry run of the library's address-range checks."""
    import torch

    import synth
    from synth import configs
    import lossless_speculative_decoding_amd as vc
    from lossless_speculative_decoding_amd import runtime
    from lossless_speculative_decoding_amd.engine import Engine, greedy_from_host, make_weights

    dry = runtime.RT.dry
    device = runtime.RT.device
    sync = runtime.RT.synchronize
    w = configs.ALL[args.config]()
    if w.compress.kind == "tokdrop" and (args.score != "attn" or args.ratio):
        import dataclasses
        ratio = args.ratio or w.compress.ratio
        spec = dataclasses.replace(w.compress, score=args.score, ratio=ratio,
                                   keep_recent=0 if args.score == "keynorm" else w.compress.keep_recent)
        name = w.name.replace(f"tokdrop{w.compress.ratio}x", f"tokdrop{ratio}x" + ("_keynorm" if args.score ==
                                                                                       "keynorm" else ""))
        w = dataclasses.replace(w, compress=spec, name=name)
    s = w.model
    ctx = list(w.ctx)
    if args.ctx:
        ctx = [args.ctx] * len(ctx)
    if args.batch:
        ctx = ctx[: args.batch]
    xs = list(w.x)[: len(ctx)]
    if not dry:
        torch.cuda.set_device(0)
    t_setup = time.perf_counter()
    n_cap = w.n_tokens
    W = make_weights(s, device=device)
    model = vc.Model(s, W, max_pos=max(ctx) + n_cap + 64)
    sampled = args.temperature is not None
    eng = Engine(model, w.compress, chunk=PREFILL_CHUNK, device=device, temperature=args.temperature, seed=args.seed)
    prefill_prof = None
    for r, (T, x) in enumerate(zip(ctx, xs)):
        p = torch.empty(T, dtype=torch.int32, device=device)
        vc.synth_ids(p, synth.S_PROMPT + r, s.vocab)
        t0 = time.perf_counter()
        if r == 0:  # request 0's prefill: live timing of its tiled GEMMs and causal attention
            vc.profile_enable((vc.VC_PROF_GEMM_TILED, vc.VC_PROF_PREFILL_ATTN))
        eng.add_request(p, x, n_cap, keep_prefill_kv=(r == 0))
        if r == 0:
            vc.profile_enable(())
            prefill_prof = {"gemm": vc.profile_read(vc.VC_PROF_GEMM_TILED),
                            "attention": vc.profile_read(vc.VC_PROF_PREFILL_ATTN), "tokens": T}
        log(f"request {r}: T={T} prefill+compress+offload {time.perf_counter() - t0:.1f}s")
    x_round = max(xs)
    eng.start(lead=args.lead or None, draft_batch=args.draft_batch or None, queue_min=args.queue_min, n_slots=args.slots,
              adaptive=args.adaptive, x_min=max(xs), fallback_after=args.fallback_after, plain_rounds=args.plain_rounds)
    t_setup = time.perf_counter() - t_setup
    log(f"setup {t_setup:.1f}s")

    # warmup (draft-attention launches recorded too, so that a counter profile of this command,
    # which sees every launch, can be compared with the algorithmic bytes of the same launches)
    kinds = (vc.VC_PROF_DRAFT_ATTN, vc.VC_PROF_VERIFY_ATTN)
    for k in kinds:
        vc.profile_read(k)
    vc.profile_enable(kinds)
    n_req = len(eng.reqs)
    # whole-decode window: from the first decoding round to every request's last token
    sync()
    t_dec0 = time.perf_counter()
    g_dec0 = sum(len(r.emitted) for r in eng.reqs)   # the prefills' first tokens
    eng.run_rounds_each(args.warmup)
    if args.adaptive:
        # the drafting horizon that still hides one request's host-row copy: L_min = ceil(t_copy / t_step),
        # t_copy at the measured pinned host-to-device rate, t_step = one batched draft step of every request
        # (timed here; the drafts it writes are overwritten by the real ones)
        import math
        eng.drain()
        from lossless_speculative_decoding_amd.engine import DONE
        live_w = [r for r in eng.reqs if r.phase != DONE]
        sync()
        t_w = time.perf_counter()
        for _ in range(4):
            eng.m.draft_step([r.req for r in live_w], eng.ws_draft)
            for r in live_w:
                r.req.draft_idx += 1
        sync()
        t_step = (time.perf_counter() - t_w) / 4
        for r in live_w:
            r.req.draft_idx = 0
        n_host_bytes = 2 * max(r.n_host for r in eng.reqs) * s.n_layers * s.n_kv_heads * s.head_dim * 2
        t_copy = n_host_bytes / (PCIE_PINNED_GBS * 1e9)
        eng.x_min = max(1, min(max(xs), math.ceil(t_copy / t_step)))
        log(f"adaptive draft length: L_min = {eng.x_min} (t_copy {t_copy * 1e3:.1f} ms, t_step {t_step * 1e3:.2f} ms)")
    eng.drain()
    warm = vc.profile_read()
    vc.profile_read(vc.VC_PROF_VERIFY_ATTN)
    # timed region
    sync()
    e0 = eng.emitted_total()
    sb0, sn0 = eng.staged_bytes, eng.stagings
    a0 = [len(r.accepts) for r in eng.reqs]
    d0, ds0 = eng.drafted, eng.draft_steps
    t0 = time.perf_counter()
    eng.run_rounds_each(args.steps)
    eng.drain()
    sync()
    secs = time.perf_counter() - t0
    vc.profile_enable(())
    prof = vc.profile_read()
    vprof = vc.profile_read(vc.VC_PROF_VERIFY_ATTN)
    emitted = eng.emitted_total() - e0
    mean_draft_batch = (eng.drafted - d0) / max(eng.draft_steps - ds0, 1)
    drafted_timed = eng.drafted - d0
    staged, n_staged = eng.staged_bytes - sb0, eng.stagings - sn0
    tok_s = emitted / secs
    accepts = [a for r, n0 in zip(eng.reqs, a0) for a in r.accepts[n0:]]
    hist = {}
    for a in accepts:
        hist[a] = hist.get(a, 0) + 1
    log(f"timed: {emitted} tokens in {secs:.2f}s = {tok_s:.2f} tok/s; mean accepted {sum(accepts)/max(len(accepts),1):.2f}")
    # the rest of the decode, to every request's token count: whole-decode tokens/s = every generated token
    # of every request / wall time from the first round to the last
    if not args.no_whole_decode:
        eng.run_to_end(progress=lambda n, t: log(f"  whole decode: {n} tokens after {t:.0f}s"))
    sync()
    dec_secs = time.perf_counter() - t_dec0
    dec_tokens = sum(min(len(r.emitted), r.n_tokens) for r in eng.reqs) - g_dec0
    dec_accepts = [a for r in eng.reqs for a in r.accepts]
    log(f"whole decode: {dec_tokens} tokens in {dec_secs:.2f}s = {dec_tokens / dec_secs:.2f} tok/s over "
        f"{len(dec_accepts)} rounds")

    att_ms = prof["ms"] / max(prof["launches"], 1)
    att_gbs = prof["bytes"] / max(prof["ms"], 1e-9) / 1e6
    all_launches = warm["launches"] + prof["launches"]
    all_bytes = (warm["bytes"] + prof["bytes"]) / max(all_launches, 1)
    traffic_ratio = pmc_traffic_ratio(w.name)
    bpl = prof["bytes"] / max(prof["launches"], 1)
    traffic = round(traffic_ratio * bpl) if traffic_ratio else None
    pcie_gbs = staged / secs / 1e9
    verify_rate = _rate(vprof, "hbm", "verification attention partials (one layer of one request)")
    if verify_rate:
        v_ratio = pmc_traffic_ratio(w.name, "attn_rows_bf16", "verify_attention")
        verify_rate["traffic"] = round(v_ratio * verify_rate["bytes_per_launch"]) if v_ratio else None
        verify_rate["traffic_over_algorithmic"] = v_ratio
    # compressed-only decoding (lossy; context): x batched draft steps of every request, no verification
    # (requests whose tail has no room for x more rows are rolled back to the last position that
    # has: this pass follows the timed region and only its rate is kept)
    live = list(eng.reqs)
    for r in live:
        r.req.n_tail = min(r.req.n_tail, r.tail_k.shape[2] - r.x - 1)
        r.req.ctx_len = r.T + r.req.n_tail
        r.req.draft_idx = 0
    sync()
    t_d = time.perf_counter()
    for _ in range(x_round):
        eng.m.draft_step([r.req for r in live], eng.ws_draft)
        for r in live:
            r.req.draft_idx = min(r.req.draft_idx + 1, r.x - 1)
    sync()
    draft_only = len(live) * x_round / (time.perf_counter() - t_d)
    # the same draft steps again with live timing of their weight-streaming GEMMs (separate
    # pass: a per-GEMM event pair is not free at these kernel lengths)
    vc.profile_read(vc.VC_PROF_GEMM_SKINNY)
    vc.profile_enable((vc.VC_PROF_GEMM_SKINNY,))
    for _ in range(x_round):
        eng.m.draft_step([r.req for r in live], eng.ws_draft)
        for r in live:
            r.req.draft_idx = min(r.req.draft_idx + 1, r.x - 1)
    sync()
    vc.profile_enable(())
    gprof = vc.profile_read(vc.VC_PROF_GEMM_SKINNY)
    for r in live:
        r.req.draft_idx = 0
    log(f"compressed-only draft decoding (lossy): {draft_only:.1f} tok/s over {len(live)} requests")

    # full-KV-from-host greedy comparator: request 0's prompt decoded again as a plain request
    # whose whole cache is on the host (after the timed region); its tokens must be the ones
    # VeriCache emitted for request 0
    r0 = eng.reqs[0]
    eng.release_host()  # the comparator needs host memory for a whole full KV
    first = torch.tensor([r0.emitted[0]], dtype=torch.int32, device=device)
    toks, bsecs = greedy_from_host(model, r0.prefill_kv, r0.T, first, args.baseline_steps, eng.ws_verify,
                                   eng.copy_stream, layered=args.comparator_staging == "layered")
    base_tok_s = args.baseline_steps / bsecs
    n_cmp = min(len(toks), len(r0.emitted) - 1)
    # sampled decoding emits another draw of the same distribution: tokens are not comparable
    base_match = None if sampled else toks[:n_cmp] == r0.emitted[1:1 + n_cmp]
    log(f"full-KV-from-host greedy: {base_tok_s:.2f} tok/s; its {n_cmp} tokens match VeriCache's: {base_match}")
    # resident full-KV greedy (context only: the workload keeps the full cache on the host): request
    # 0 alone with its whole cache in HBM, one vc_verify row per token appended in place
    from lossless_speculative_decoding_amd._vc import Req
    n_res = min(len(r0.emitted), r0.n_tokens) - 1   # every token request 0 emitted after its first
    cap = r0.T + n_res + 1
    kd = torch.empty(s.n_layers, s.n_kv_heads, cap, s.head_dim, dtype=r0.prefill_kv[0].dtype, device=device)
    vd = torch.empty_like(kd)
    if not dry:  # data only (a dry run computes nothing)
        kd[:, :, :r0.T].copy_(r0.prefill_kv[0][:, :, :r0.T])
        vd[:, :, :r0.T].copy_(r0.prefill_kv[1][:, :, :r0.T])
    del r0.prefill_kv
    res_rows = torch.empty(n_res + 1, dtype=torch.int32, device=device)
    res_rows[:1].copy_(first)
    vc.debug_register(kd, vd, res_rows, eng.ws_verify)
    rreq = Req(ctx_len=r0.T)
    row_b = s.head_dim * kd.element_size()
    sync()
    t_r = time.perf_counter()
    for i in range(n_res):
        rreq.ctx_len = r0.T + i
        off = rreq.ctx_len * row_b
        model.verify_raw(rreq, kd.data_ptr(), vd.data_ptr(), cap, res_rows.data_ptr() + 4 * i, 1,
                         res_rows.data_ptr() + 4 * (i + 1), kd.data_ptr() + off, vd.data_ptr() + off, cap, eng.ws_verify)
    sync()
    res_tok_s = n_res / (time.perf_counter() - t_r)
    n_rc = min(n_res, len(r0.emitted) - 1)
    res_match = None if sampled else res_rows[1:1 + n_rc].tolist() == r0.emitted[1:1 + n_rc]
    del kd, vd
    log(f"resident full-KV greedy (one request, context): {res_tok_s:.1f} tok/s; tokens match VeriCache's: {res_match}")

    cpu = None
    if not args.no_cpu_baseline and not dry:
        keep = ctx[0] // w.compress.ratio if w.compress.kind == "tokdrop" else ctx[0]
        cpu = cpu_baseline(s, ctx[0], keep)
        log(f"cpu baseline {cpu['value']:.4f} {cpu['unit']}")

    return {
        "metric": "lossless decode tokens/s at 1 GPU; draft-attn HBM GB/s vs peak",
        "value": round(tok_s, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1000 * secs / args.steps, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and uniform prompt ids)",
        "decoding": "greedy" if not sampled else f"sampled, temperature {args.temperature}, seed {args.seed} "
                                                 "(speculative rejection sampling)",
        "config": {"workload": w.name, "batch": len(ctx), "ctx": ctx if len(set(ctx)) > 1 else ctx[0],
                   "x": xs if len(set(xs)) > 1 else xs[0],
                   "compress": w.compress.kind + ("" if w.compress.kind != "tokdrop" else
                                                  f" {w.compress.ratio}x by {w.compress.score}"),
                   "full_kv": "pinned host for the rows the GPU does not hold exactly, staged over PCIe per "
                              "verification",
                   "timed_rounds": f"verification rounds {args.warmup + 1}..{args.warmup + args.steps} of every "
                                   f"request, up to its {w.n_tokens}th token"},
        "roofline": {"bound": "hbm", "kernel": "draft attention partials (all layers of a draft step)",
                     "achieved": round(att_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(att_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "traffic_over_algorithmic": traffic_ratio,
                     "avg_launch_ms": round(att_ms, 5), "launches": prof["launches"],
                     "bytes_per_launch": round(prof["bytes"] / max(prof["launches"], 1)),
                     "partial_bytes_per_launch": round(prof["aux_bytes"] / max(prof["launches"], 1)),
                     "bytes_per_launch_incl_warmup": round(all_bytes), "launches_incl_warmup": all_launches},
        "verify_attention": verify_rate,
        "gemm_decode": _rate(gprof, "hbm", f"projection and LM-head GEMMs of {len(live)}-request draft steps "
                                           "(weight streaming)"),
        "gemm_prefill": _rate(prefill_prof["gemm"], "mfma", f"projection GEMMs of request 0's prefill "
                                                             f"({prefill_prof['tokens']} tokens, {PREFILL_CHUNK}-row chunks)"),
        "attention_prefill": _rate(prefill_prof["attention"], "mfma", "causal attention of request 0's prefill "
                                                                      f"({PREFILL_CHUNK}-row chunks)"),
        "pcie": {"bound": "pcie", "achieved": round(pcie_gbs, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                 "frac": round(pcie_gbs / PCIE_PEAK_GBS, 4), "stagings": n_staged,
                 "bytes_per_staging": round(staged / max(n_staged, 1)),
                 "note": "host rows staged for verification in the timed region / its wall time"},
        "full_kv_from_host_tok_s": round(base_tok_s, 3),
        "full_kv_from_host_tokens_match": base_match,
        "full_kv_from_host_staging": args.comparator_staging,
        "resident_full_kv_greedy_tok_s": round(res_tok_s, 2),
        "resident_full_kv_note": "context only: request 0 alone with its whole cache in HBM (the workload keeps it "
                                 "on the host); tokens match VeriCache's: " + str(res_match),
        "speedup_vs_full_kv_from_host": round(tok_s / base_tok_s, 3),
        "scheduler": {"draft_batch": eng.draft_batch, "queue_min": eng.queue_min, "lead": eng.lead,
                      "slots": len(eng.slots), "adaptive": args.adaptive,
                      "x_min": eng.x_min if args.adaptive else None,
                      "fallback_after": args.fallback_after if args.adaptive else None,
                      "plain_rounds": args.plain_rounds if args.adaptive and args.fallback_after else None,
                      "plain_round_share": round(sum(1 for r in eng.reqs for g in r.x_hist if g == 0) /
                                                 max(sum(len(r.x_hist) for r in eng.reqs), 1), 4),
                      "drafts_per_round": round(drafted_timed / max(len(accepts), 1), 2),
                      "mean_requests_per_draft_step": round(mean_draft_batch, 2)},
        "whole_decode": None if args.no_whole_decode else {"tokens_per_s": round(dec_tokens / dec_secs, 3), "tokens": dec_tokens,
                         "seconds": round(dec_secs, 2), "rounds": len(dec_accepts),
                         "mean_accepted_per_round": round(sum(dec_accepts) / max(len(dec_accepts), 1), 3),
                         "note": f"every generated token of every request ({w.n_tokens} per request, the first "
                                 "from the prefill excluded) over the wall time of the whole decode, warmup and "
                                 "timed rounds included"},
        "mean_accepted_per_round": round(sum(accepts) / max(len(accepts), 1), 3),
        "rounds": len(accepts),
        "rounds_per_s": round(len(accepts) / secs, 3),
        "accept_hist": {str(k): hist[k] for k in sorted(hist)},
        "compressed_only_draft_tok_s": round(draft_only, 2),
        "cpu_baseline": cpu,
    }


def run_remote_prefix(args) -> dict:
    """Remote prefix caching (the second serving setting of "VeriCache: Making Lossy KV Compression
    Exact", "Verifying Without Giving Back the Speedup"; the study note's "实践案例" case 3).  Every
    request's prompt cache is precomputed (untimed) and kept in host memory standing in for remote
    storage behind a slow link of --remote-link GB/s (the page's example: about 3 GB/s from object
    storage).  VeriCache ships only the compressed caches over that link and starts drafting a request
    as soon as its cache has landed; verification reads the exact rows over PCIe as in the long-context
    loop (the storage side's fast link).  The comparator ships each full prompt cache over the same slow
    link and decodes the request with it resident as soon as it has landed.  Both decode every request
    to --remote-tokens tokens; reported: time to the first generated token (the first after the
    prefix's own next token) per request and tokens/s over the whole job, shipping included, from the
    first byte on the link.  Tokens must be equal."""
    import torch

    import synth
    from synth import configs
    import lossless_speculative_decoding_amd as vc
    from lossless_speculative_decoding_amd._vc import Req
    from lossless_speculative_decoding_amd.engine import Engine, NonFiniteLogits, make_weights
    from lossless_speculative_decoding_amd.remote import SlowLink

    sync = torch.cuda.synchronize
    w = configs.ALL[args.config]()
    s = w.model
    ctx = list(w.ctx)[: args.batch or None]
    xs = list(w.x)[: len(ctx)]
    n_tok = args.remote_tokens
    torch.cuda.set_device(0)
    W = make_weights(s)
    model = vc.Model(s, W, max_pos=max(ctx) + n_tok + 64)
    eng = Engine(model, w.compress, chunk=PREFILL_CHUNK)
    for r, (T, x) in enumerate(zip(ctx, xs)):
        p = torch.empty(T, dtype=torch.int32, device="cuda")
        vc.synth_ids(p, synth.S_PROMPT + r, s.vocab)
        eng.add_request(p, x, n_tok, keep_prefill_kv=True)
    # the remote store (pageable host memory): compressed caches and full prompt caches; the device
    # copies of the compressed caches are wiped so that only shipped bytes can serve a draft
    import ctypes
    comp_store, comp_host, full_store = [], [], []
    for r in eng.reqs:
        # pinned memory of the exact size (the caching host allocator would round 2.15 GB up to 4 GB)
        hb = vc.HostBuffer(r.comp.numel())
        comp_host.append(hb)
        comp_store.append(torch.frombuffer((ctypes.c_uint8 * r.comp.numel()).from_address(hb.data_ptr()),
                                           dtype=torch.uint8))
        comp_store[-1].copy_(r.comp)
        full_store.append((r.prefill_kv[0].cpu(), r.prefill_kv[1].cpu()))
        r.comp.zero_()
        del r.prefill_kv
    torch.cuda.empty_cache()
    sync()
    comp_bytes = sum(c.numel() for c in comp_store)
    full_bytes = sum(k.numel() * k.element_size() * 2 for k, _ in full_store)
    log(f"remote store: {comp_bytes / 1e9:.2f} GB compressed, {full_bytes / 1e9:.2f} GB full; link "
        f"{args.remote_link} GB/s")

    # ---- VeriCache: compressed caches over the slow link (pinned store, chunks issued from the
    # scheduler's own loop), drafting as each lands
    link = SlowLink(args.remote_link)
    evs = link.start([(comp_store[i], r.comp) for i, r in enumerate(eng.reqs)])
    for r, e in zip(eng.reqs, evs):
        r.ready = e
    eng.start(adaptive=args.adaptive, x_min=max(1, min(xs) // 2), fallback_after=args.fallback_after,
              plain_rounds=args.plain_rounds)
    eng.run_to_end(progress=lambda n, t: log(f"  VeriCache: {n} tokens after {t:.0f}s"))
    link.wait()
    sync()
    t_vc = time.perf_counter() - link.t0
    vc_ttft = [round(r.t_first - link.t0, 3) for r in eng.reqs]
    vc_tokens = [r.emitted[:n_tok] for r in eng.reqs]
    n_gen = sum(len(t) - 1 for t in vc_tokens)
    accepts = [a for r in eng.reqs for a in r.accepts]
    vc_arrival = [round(a, 3) for a in link.arrival]
    log(f"VeriCache: {n_gen} tokens in {t_vc:.2f}s = {n_gen / t_vc:.2f} tok/s; first token after "
        f"{vc_ttft[0]:.2f}s (request 0) .. {max(vc_ttft):.2f}s; caches landed at {vc_arrival}")
    eng.release_host()
    del eng, evs, comp_store
    for hb in comp_host:
        hb.free()
    torch.cuda.empty_cache()

    # ---- full KV first: each full prompt cache over the slow link, then resident greedy decoding
    L, Hkv, D = s.n_layers, s.n_kv_heads, s.head_dim
    bufs = []
    for T in ctx:
        bk = torch.empty(L, Hkv, T + n_tok, D, dtype=torch.bfloat16 if s.dtype == "bf16" else torch.float32,
                         device="cuda")
        bufs.append((bk, torch.empty_like(bk)))
    jobs = []
    for (k, v), (bk, bv), T in zip(full_store, bufs, ctx):
        jobs += [(k, bk[:, :, :T]), (v, bv[:, :, :T])]
    ws = model.workspace(1, max(ctx) + n_tok)
    link2 = SlowLink(args.remote_link)
    evs2 = link2.ship(jobs)
    fk_ttft, fk_tokens = [], []
    for i, ((bk, bv), T) in enumerate(zip(bufs, ctx)):
        evs2[2 * i + 1].wait()
        if link2.error is not None:
            raise link2.error
        out = torch.empty(n_tok, dtype=torch.int32, device="cuda")
        out[:1].fill_(vc_tokens[i][0])
        cap = T + n_tok
        req = Req(ctx_len=T)
        row = D * bk.element_size()
        for j in range(1, n_tok):
            req.ctx_len = T + j - 1
            off = req.ctx_len * row
            model.verify_raw(req, bk.data_ptr(), bv.data_ptr(), cap, out.data_ptr() + 4 * (j - 1), 1,
                             out.data_ptr() + 4 * j, bk.data_ptr() + off, bv.data_ptr() + off, cap, ws)
            if j == 1:
                sync()
                fk_ttft.append(round(time.perf_counter() - link2.t0, 3))
        fk_tokens.append(out.tolist())
        log(f"  full KV first: request {i} done after {time.perf_counter() - link2.t0:.1f}s")
    link2.wait()
    sync()
    t_fk = time.perf_counter() - link2.t0
    if min(min(t) for t in fk_tokens) < 0:
        raise NonFiniteLogits("full-KV-first decoding wrote token -1")
    match = fk_tokens == vc_tokens
    log(f"full KV first: {n_gen} tokens in {t_fk:.2f}s = {n_gen / t_fk:.2f} tok/s; first token after "
        f"{fk_ttft[0]:.2f}s .. {max(fk_ttft):.2f}s; tokens equal VeriCache's: {match}")
    return {
        "metric": "remote prefix caching: tokens/s over the whole job, cache shipping included",
        "value": round(n_gen / t_vc, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and uniform prompt ids)",
        "config": {"workload": w.name + f"_remote{args.remote_link:g}gbps_{n_tok}tok", "batch": len(ctx),
                   "ctx": ctx[0] if len(set(ctx)) == 1 else ctx, "link_gbps": args.remote_link,
                   "tokens_per_request": n_tok, "adaptive": args.adaptive,
                   "fallback_after": args.fallback_after if args.adaptive else None,
                   "link": "slow link emulated by wall-clock-paced host-to-device copies (VeriCache: from a pinned "
                           "store, chunks issued by the scheduler's loop; full KV first: from pageable memory on a "
                           "worker thread)"},
        "shipped_bytes": {"vericache": comp_bytes, "full_kv_first": full_bytes},
        "vericache": {"seconds": round(t_vc, 3), "tokens_per_s": round(n_gen / t_vc, 3), "ttft_s": vc_ttft,
                      "caches_landed_s": vc_arrival,
                      "mean_accepted_per_round": round(sum(accepts) / max(len(accepts), 1), 3),
                      "rounds": len(accepts)},
        "full_kv_first": {"seconds": round(t_fk, 3), "tokens_per_s": round(n_gen / t_fk, 3), "ttft_s": fk_ttft,
                          "caches_landed_s": [round(link2.arrival[2 * i + 1], 3) for i in range(len(ctx))]},
        "speedup_whole_job": round(t_fk / t_vc, 3),
        "speedup_first_token": round(fk_ttft[0] / vc_ttft[0], 3),
        "tokens_match": match,
    }


def bounds_replay(args):
    """Replay the workload's exact sequence of library calls on the CPU with the library's
    address-range checks (vc_debug_mode VC_DEBUG_DRY): every launch and copy states the byte
    ranges it can touch, each must lie inside a buffer the caller or the library allocated (host
    memory stands in for device memory, mapped lazily), and nothing runs.  Accept counts come
    from a seeded policy that accepts every draft in every other round (the fastest-growing
    tails).  Prints the checks made; exits non-zero at the first range outside every buffer."""
    import lossless_speculative_decoding_amd as vc
    from lossless_speculative_decoding_amd import runtime
    # "collapse": runs of rounds that keep no draft between runs that keep all (plain rounds then occur
    # under --adaptive --fallback-after); default: every other round keeps all, the others a seeded count
    policy = (lambda idx, rnd, x: 0 if (rnd // 5) % 2 else x) if args.replay_policy == "collapse" else None
    runtime.use(runtime.DryRT(seed=0, accept_policy=policy))
    vc.debug_mode(vc.VC_DEBUG_DRY)
    args.no_cpu_baseline = True
    t0 = time.perf_counter()
    try:
        res = run_model_workload(args)
    except vc._vc.VCError as e:
        st = vc.debug_stats()
        print(json.dumps({"bounds_replay": args.config, "ok": False, "error": str(e), **st}), flush=True)
        sys.exit(1)
    st = vc.debug_stats()
    print(json.dumps({"bounds_replay": args.config, "ok": st["violations"] == 0, "seconds": round(time.perf_counter()
                                                                                                 - t0, 1),
                      "plain_round_share": res["scheduler"]["plain_round_share"], **st}), flush=True)
    sys.exit(0 if st["violations"] == 0 else 1)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16, help="timed verification rounds per request")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="llama8b_tokdrop",
                    choices=["llama8b_tokdrop", "llama8b_q2", "llama8b_mixed", "gqa_layer"])
    ap.add_argument("--ctx", type=int, default=0, help="override the prompt length (diagnostics only)")
    ap.add_argument("--bits", type=int, default=0, help="gqa_layer: code width of the quantized cache (2, 3, 4)")
    ap.add_argument("--group", type=int, default=0, help="gqa_layer: quantization group (64, 128)")
    ap.add_argument("--batch", type=int, default=0, help="override the batch (diagnostics only)")
    ap.add_argument("--baseline-steps", type=int, default=16)
    ap.add_argument("--comparator-staging", choices=["layered", "whole"], default="layered",
                    help="full-KV-from-host comparator: stage layer by layer with each layer's attention waiting "
                         "only for its own layer (default), or stage all layers before each verification")
    ap.add_argument("--draft-batch", type=int, default=0,
                    help="requests yet to draft wait for a batch this large while --queue-min drafted requests are "
                         "queued for verification (0: all the requests; 1: draft as soon as possible)")
    ap.add_argument("--queue-min", type=int, default=1)
    ap.add_argument("--lead", type=int, default=0, help="draft steps before a request's last draft at which its "
                    "host rows start to stage (0: as soon as its drafting has begun)")
    ap.add_argument("--slots", type=int, default=3, help="device staging slots")
    ap.add_argument("--score", choices=["attn", "keynorm"], default="attn",
                    help="token-drop ranking: observed attention (the workload's) or key norm (the pages' example "
                         "compressor: no recent window)")
    ap.add_argument("--ratio", type=int, default=0, help="token-drop compression ratio (0: the workload's)")
    ap.add_argument("--adaptive", action="store_true",
                    help="per-request draft length between L_min = ceil(t_copy / t_step) (measured in the warmup) "
                         "and the workload's x: doubled after an all-accepted round, a + 1 after a rejection")
    ap.add_argument("--fallback-after", type=int, default=0,
                    help="with --adaptive: after this many consecutive rounds that keep no draft, decode plainly "
                         "(no drafts) for --plain-rounds rounds (0: never)")
    ap.add_argument("--plain-rounds", type=int, default=8)
    ap.add_argument("--temperature", type=float, default=None,
                    help="sampled decoding at this temperature with speculative rejection sampling (default: greedy)")
    ap.add_argument("--seed", type=int, default=0, help="generator key of sampled decoding")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-whole-decode", action="store_true",
                    help="skip decoding the rest of every request after the timed rounds (the whole-decode rate)")
    ap.add_argument("--check-bounds", action="store_true",
                    help="check every launch's and copy's byte ranges against the buffers allocated for it before "
                         "it runs on the GPU (an error instead of a launch outside them)")
    ap.add_argument("--bounds-replay", action="store_true",
                    help="no GPU work: replay the workload's sequence of library calls on the CPU with every "
                         "launch's byte ranges checked against the buffers allocated for it")
    ap.add_argument("--remote-link", type=float, default=0.0,
                    help="remote prefix caching: ship caches over a slow link of this many GB/s (0: off)")
    ap.add_argument("--remote-tokens", type=int, default=64, help="remote prefix caching: tokens per request")
    ap.add_argument("--replay-policy", choices=["grow", "collapse"], default="grow",
                    help="accept counts a bounds replay assumes (collapse: runs of rounds that keep no draft)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference kernel that scales "
                         "the HBM byte counters of a profile)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty(1 << 30, dtype=torch.int8, device="cuda")
        for _ in range(5):
            dst.copy_(src)  # uint8 -> int8: an elementwise kernel that reads and writes 1 GiB (not a DMA)
        torch.cuda.synchronize()
        log("copied 5 x 1 GiB")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (requests would be sharded across "
              "GPUs by request, each GPU running this same loop)", file=sys.stderr)
        sys.exit(2)

    if args.config == "gqa_layer":
        bench_layer(args)
        return

    if args.config in DISABLED and not args.bounds_replay:
        sys.exit(f"bench.py: workload {args.config} is disabled: {DISABLED[args.config]}")
    if args.remote_link > 0:
        print(json.dumps(run_remote_prefix(args)), flush=True)
        return
    if args.bounds_replay:
        bounds_replay(args)
        return
    if args.check_bounds:
        import lossless_speculative_decoding_amd as vc
        vc.debug_mode(vc.VC_DEBUG_CHECK)
    line = run_model_workload(args)
    if args.check_bounds:
        line["bounds_checks"] = vc.debug_stats()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
