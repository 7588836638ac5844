"""Thin torch-facing wrappers over the C ABI (same names as include/vc.h).

Each wrapper converts torch tensors to device pointers and the current torch
stream to a hipStream_t, allocates outputs/workspaces with torch, and calls
the library.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _vc, runtime
from ._vc import (VC_BF16, VC_F32, VC_PROF_DRAFT_ATTN, VC_PROF_GEMM_SKINNY, VC_PROF_GEMM_TILED,
                  VC_PROF_PREFILL_ATTN, VC_PROF_VERIFY_ATTN, VC_QUANT, VC_SCORE_ATTN, VC_SCORE_KEYNORM, VC_TOKDROP,
                  VC_DEBUG_CHECK, VC_DEBUG_DRY, VC_DEBUG_OFF, AttnDesc, AttnDraftReq, DebugStats,
                  CompressDesc, CompressLayout, ModelDesc, ProfileStats, Req, Sampler, Weights, call,
                  VC_DRAW_ACCEPT, VC_DRAW_DRAFT, VC_DRAW_TARGET)

__all__ = ["VC_BF16", "VC_F32", "VC_QUANT", "VC_TOKDROP", "VC_SCORE_ATTN", "VC_SCORE_KEYNORM", "CompressDesc", "Req", "Model", "compress_desc",
           "compress_layout", "vc_compress", "vc_linear", "vc_attn_draft", "vc_attn_verify", "synth_xavier",
           "synth_normal_heads", "synth_ids", "synth_fill", "stream_handle", "torch_dtype", "elem_bytes",
           "profile_enable", "profile_read", "HostBuffer", "PageableBuffer", "VC_PROF_DRAFT_ATTN",
           "VC_PROF_VERIFY_ATTN", "VC_PROF_GEMM_SKINNY", "VC_PROF_GEMM_TILED", "VC_PROF_PREFILL_ATTN",
           "VC_DEBUG_OFF", "VC_DEBUG_CHECK", "VC_DEBUG_DRY", "debug_mode", "debug_register", "debug_stats",
           "Sampler", "VC_DRAW_DRAFT", "VC_DRAW_ACCEPT", "VC_DRAW_TARGET", "vc_sample", "spec_ws_size",
           "vc_spec_sample"]

_DBG = False   # address-range checks on: every tensor handed to the library is registered
_DRY = False   # dry run: host tensors stand in for device tensors


def stream_handle(s=None) -> int:
    s = s or runtime.RT.current_stream()
    return s.cuda_stream


def debug_register(*tensors) -> None:
    """Register the storage of each tensor as a buffer the library may touch (range checks)."""
    if not _DBG:
        return
    for t in tensors:
        if t is not None:
            st = t.untyped_storage()
            call("vc_debug_register", st.data_ptr(), st.nbytes())


def debug_mode(mode: int) -> None:
    """VC_DEBUG_OFF, VC_DEBUG_CHECK (every launch's byte ranges checked against registered
    buffers first) or VC_DEBUG_DRY (checked, then nothing launched; host tensors stand in for
    device tensors).  In dry mode select runtime.DryRT() as well."""
    global _DBG, _DRY
    call("vc_debug_mode", mode)
    _DBG, _DRY = mode != VC_DEBUG_OFF, mode == VC_DEBUG_DRY


def debug_stats(reset: bool = False) -> dict:
    st = DebugStats()
    call("vc_debug_stats_read", C.byref(st), int(reset))
    return {"launches": st.launches, "ranges": st.ranges, "violations": st.violations,
            "pinned_bytes": st.pinned_bytes, "pinned_peak": st.pinned_peak}


def ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda and not _DRY:
        raise ValueError("expected a device tensor")
    debug_register(t)
    return t.data_ptr()


def torch_dtype(vc_dtype: int):
    return torch.bfloat16 if vc_dtype == VC_BF16 else torch.float32


def elem_bytes(vc_dtype: int) -> int:
    return 2 if vc_dtype == VC_BF16 else 4


# ---------------------------------------------------------------- compression
def compress_desc(kind: int, n_layers: int, n_q_heads: int, n_kv_heads: int, head_dim: int, seq_len: int,
                  dtype: int, src_cap: int | None = None, bits: int = 0, group: int = 0, keep_total: int = 0,
                  keep_recent: int = 64, obs_window: int = 32, score: int = 0) -> CompressDesc:
    return CompressDesc(kind=kind, bits=bits, group=group, keep_total=keep_total, keep_recent=keep_recent,
                        obs_window=obs_window, n_layers=n_layers, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                        head_dim=head_dim, seq_len=seq_len, dtype=dtype, src_cap=src_cap or seq_len, score=score)


def compress_layout(d: CompressDesc) -> CompressLayout:
    lay = CompressLayout()
    call("vc_compress_layout_of", C.byref(d), C.byref(lay))
    return lay


def vc_compress(d: CompressDesc, k: torch.Tensor, v: torch.Tensor, q_obs: torch.Tensor | None = None,
                out: torch.Tensor | None = None) -> torch.Tensor:
    ob, wb = C.c_size_t(), C.c_size_t()
    call("vc_compress_size", C.byref(d), C.byref(ob), C.byref(wb))
    if out is None:  # zeroed so that the bytes between sections are defined (not in a dry run)
        out = (torch.empty if _DRY else torch.zeros)(ob.value, dtype=torch.uint8, device=k.device)
    ws = torch.empty(max(wb.value, 256), dtype=torch.uint8, device=k.device)
    call("vc_compress", C.byref(d), ptr(k), ptr(v), ptr(q_obs), ptr(out), out.numel(), ptr(ws), ws.numel(),
         stream_handle())
    return out


# ---------------------------------------------------------------- one projection GEMM
def vc_linear(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """y[M][N] float32 = x[M][K] w[N][K]^T (bf16 or float32 operands, float32 sums)."""
    M, K = x.shape
    N = w.shape[0]
    assert w.shape == (N, K) and w.dtype == x.dtype and x.is_contiguous() and w.is_contiguous()
    y = torch.empty(M, N, dtype=torch.float32, device=x.device)
    dt = VC_BF16 if x.dtype == torch.bfloat16 else VC_F32
    call("vc_linear", ptr(x), ptr(w), ptr(y), M, N, K, dt, stream_handle())
    return y


# ---------------------------------------------------------------- single-layer attention
def vc_attn_draft(d: AttnDesc, comps, cds, tails_k, tails_v, n_tail, q: torch.Tensor) -> torch.Tensor:
    n = len(comps)
    reqs = (AttnDraftReq * n)()
    keep = []
    for r in range(n):
        cd = cds[r]
        keep.append(cd)
        tk, tv = tails_k[r], tails_v[r]
        reqs[r] = AttnDraftReq(comp=ptr(comps[r]), cd=C.pointer(cd), tail_k=ptr(tk), tail_v=ptr(tv),
                               tail_cap=tk.shape[-2] if tk is not None else 0, n_tail=n_tail[r])
    out = torch.empty(q.shape, dtype=torch_dtype(d.out_dtype), device=q.device)
    wb = C.c_size_t()
    max_keys = max(compress_layout(cd).n_main + compress_layout(cd).n_resid for cd in cds) + max(n_tail) + 1
    call("vc_attn_ws_size", C.byref(d), n, 1, max_keys, C.byref(wb))
    ws = torch.empty(wb.value, dtype=torch.uint8, device=q.device)
    call("vc_attn_draft", C.byref(d), reqs, n, ptr(q), ptr(out), ptr(ws), ws.numel(), stream_handle())
    return out


def vc_attn_verify(d: AttnDesc, q: torch.Tensor, staged_k, staged_v, ctx, tails_k, tails_v, n_rows: int,
                   split_len: int = 0) -> torch.Tensor:
    """q [n][n_rows][Hq][D]; staged_* lists of [Hkv][cap][D]; tails_* lists of [Hkv][tcap][D]."""
    n = q.shape[0]
    P = C.c_void_p * n
    sk = P(*[ptr(t) for t in staged_k])
    sv = P(*[ptr(t) for t in staged_v])
    tk = P(*[ptr(t) for t in tails_k])
    tv = P(*[ptr(t) for t in tails_v])
    cx = (C.c_int32 * n)(*ctx)
    out = torch.empty(q.shape, dtype=torch_dtype(d.out_dtype), device=q.device)
    d2 = AttnDesc(d.n_q_heads, d.n_kv_heads, d.head_dim, d.dtype, split_len or d.split_len, d.out_dtype)
    split = d2.split_len or 1024
    S = -(-(max(ctx) + n_rows) // split)
    nbytes = n * n_rows * d.n_q_heads * S * (d.head_dim + 2) * 4 + 256
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    call("vc_attn_verify", C.byref(d2), n, ptr(q), sk, sv, staged_k[0].shape[-2], cx, tk, tv, tails_k[0].shape[-2],
         n_rows, ptr(out), ptr(ws), ws.numel(), stream_handle())
    return out


# ---------------------------------------------------------------- synthetic inputs (GPU generator)
def synth_xavier(t: torch.Tensor, stream_id: int, fan_in: int, fan_out: int, seed: int = 0, start: int = 0):
    dt = VC_BF16 if t.dtype == torch.bfloat16 else VC_F32
    call("vc_synth_xavier", ptr(t), dt, t.numel(), stream_id, seed, start, fan_in, fan_out, stream_handle())
    return t


def synth_normal_heads(t: torch.Tensor, stream_id: int, outl: torch.Tensor | None = None, outl_scale: float = 10.0,
                       seed: int = 0):
    B, H, rows, D = t.shape
    n_outl = outl.shape[-1] if outl is not None else 0
    call("vc_synth_normal_heads", ptr(t), B, H, rows, D, stream_id, seed, ptr(outl), n_outl, outl_scale,
         stream_handle())
    return t


def synth_ids(t: torch.Tensor, stream_id: int, vocab: int, seed: int = 0):
    call("vc_synth_ids", ptr(t), t.numel(), stream_id, seed, vocab, stream_handle())
    return t


def synth_fill(t: torch.Tensor, value: float):
    dt = VC_BF16 if t.dtype == torch.bfloat16 else VC_F32
    call("vc_synth_fill", ptr(t), dt, t.numel(), value, stream_handle())
    return t


# ---------------------------------------------------------------- model
class Model:
    """A vc_model over caller-owned torch weight tensors (kept alive here)."""

    def __init__(self, shape, weights: dict, max_pos: int):
        s = shape
        self.shape = s
        self.dtype = VC_BF16 if s.dtype == "bf16" else VC_F32
        self.eb = elem_bytes(self.dtype)
        self.w = weights
        self.desc = ModelDesc(s.n_layers, s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ffn, s.vocab,
                              self.dtype, s.rope_theta, s.eps, max_pos)
        self.cw = Weights(*[ptr(weights[k]) for k in ("embed", "lm_head", "norm_final", "norm_attn", "norm_ffn",
                                                      "w_qkv", "w_o", "w_gu", "w_down")])
        h = C.c_void_p()
        call("vc_model_create", C.byref(self.desc), C.byref(self.cw), stream_handle(), C.byref(h))
        self.h = h

    def close(self):
        if self.h:
            call("vc_model_destroy", self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def ws_size(self, max_rows: int, max_keys: int) -> int:
        b = C.c_size_t()
        call("vc_ws_size", self.h, max_rows, max_keys, C.byref(b))
        return b.value

    def workspace(self, max_rows: int, max_keys: int, device="cuda") -> torch.Tensor:
        return torch.empty(self.ws_size(max_rows, max_keys), dtype=torch.uint8, device=device)

    def prefill(self, tokens: torch.Tensor, k_out, v_out, q_obs, W: int, g0: torch.Tensor, ws: torch.Tensor,
                chunk: int, last_logits=None):
        call("vc_prefill", self.h, ptr(tokens), tokens.numel(), ptr(k_out), ptr(v_out), k_out.shape[-2],
             ptr(q_obs), W, ptr(g0), ptr(last_logits), chunk, ptr(ws), ws.numel(), stream_handle())

    def draft_step(self, reqs, ws: torch.Tensor, logits=None):
        n = len(reqs)
        arr = (Req * n)(*reqs)
        call("vc_draft_step", self.h, arr, n, ptr(logits), ptr(ws), ws.numel(), stream_handle())
        return arr

    def draft_step_sampled(self, reqs, samplers, probs, ws: torch.Tensor, logits=None):
        """vc_draft_step_sampled: samplers, one _vc.Sampler per request; probs, one fp32
        device tensor [>= x][vocab] per request (row draft_idx is written)."""
        n = len(reqs)
        arr = (Req * n)(*reqs)
        sm = (Sampler * n)(*samplers)
        pp = (C.c_void_p * n)(*[ptr(p) for p in probs])
        call("vc_draft_step_sampled", self.h, arr, n, sm, pp, ptr(logits), ptr(ws), ws.numel(), stream_handle())
        return arr

    def draft_step_static(self, reqs, logits=None):
        """vc_draft_step with the library's static workspace (no allocation)."""
        n = len(reqs)
        arr = (Req * n)(*reqs)
        call("vc_draft_step_static", self.h, arr, n, ptr(logits), stream_handle())
        return arr

    def verify_raw(self, req: Req, staged_k: int, staged_v: int, staged_cap: int, tok: int, n_rows: int, out: int,
                   vtail_k: int, vtail_v: int, vtail_cap: int, ws: torch.Tensor, logits: int | None = None):
        call("vc_verify", self.h, C.byref(req), staged_k, staged_v, staged_cap, tok, n_rows, out, logits, vtail_k,
             vtail_v, vtail_cap, ptr(ws), ws.numel(), stream_handle())

    def verify_layered_raw(self, req: Req, staged_k: int, staged_v: int, staged_cap: int, tok: int, n_rows: int,
                           out: int, vtail_k: int, vtail_v: int, vtail_cap: int, ws: torch.Tensor, layer_ready,
                           logits: int | None = None):
        """vc_verify_layered: layer l's attention waits for layer_ready[l] (one event per layer)."""
        evs = (C.c_void_p * len(layer_ready))(*[e.cuda_event for e in layer_ready])
        call("vc_verify_layered", self.h, C.byref(req), staged_k, staged_v, staged_cap, tok, n_rows, out, logits,
             vtail_k, vtail_v, vtail_cap, ptr(ws), ws.numel(), evs, stream_handle())

    def verify(self, req: Req, staged_k, staged_v, tok: torch.Tensor, n_rows: int, out: torch.Tensor, vtail_k,
               vtail_v, ws: torch.Tensor, logits=None):
        scap = staged_k.shape[-2] if staged_k is not None else 0
        self.verify_raw(req, ptr(staged_k), ptr(staged_v), scap, ptr(tok), n_rows, ptr(out), ptr(vtail_k),
                        ptr(vtail_v), vtail_k.shape[-2], ws, ptr(logits))

    def accept(self, req: Req, verified, x: int, vtail_k, vtail_v, result: torch.Tensor):
        call("vc_accept", self.h, C.byref(req), ptr(verified), x, ptr(vtail_k), ptr(vtail_v), vtail_k.shape[-2],
             ptr(result), stream_handle())

    def commit(self, req: Req, a: int, vtail_k, vtail_v, after_event=None, copy_stream=None):
        ev = after_event.cuda_event if after_event is not None else None
        call("vc_commit", self.h, C.byref(req), a, ptr(vtail_k), ptr(vtail_v), vtail_k.shape[-2], ev,
             stream_handle(copy_stream))

    def offload(self, req: Req, k_dev, v_dev, T: int, l0: int | None = None, l1: int | None = None):
        if l0 is None:
            call("vc_offload", self.h, C.byref(req), ptr(k_dev), ptr(v_dev), k_dev.shape[-2], T, stream_handle())
        else:
            call("vc_offload_layers", self.h, C.byref(req), ptr(k_dev), ptr(v_dev), k_dev.shape[-2], T, l0, l1,
                 stream_handle())

    def stage(self, req: Req, slot_k, slot_v, l0: int, l1: int, copy_stream=None):
        call("vc_stage", self.h, C.byref(req), ptr(slot_k), ptr(slot_v), slot_k.shape[-2], l0, l1,
             stream_handle(copy_stream))


# ---------------------------------------------------------------- sampled decoding
def vc_sample(logits: torch.Tensor, samplers, pos, purpose: int, out: torch.Tensor | None = None,
              probs: torch.Tensor | None = None) -> torch.Tensor:
    """One draw per row of logits [n][vocab] (fp32, device); samplers: one Sampler per row;
    pos: the position of each row's token.  Returns the int32 tokens."""
    n, V = logits.shape
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=logits.device)
    sm = (Sampler * n)(*samplers)
    ps = (C.c_int64 * n)(*[int(p) for p in pos])
    call("vc_sample", ptr(logits), n, V, sm, ps, purpose, ptr(out), ptr(probs), stream_handle())
    return out


def spec_ws_size(x: int) -> int:
    b = C.c_size_t()
    call("vc_spec_ws_size", x, C.byref(b))
    return b.value


def vc_spec_sample(logits_t: torch.Tensor, probs_d: torch.Tensor | None, draft: torch.Tensor | int, x: int,
                   sampler, pos0: int, verified: torch.Tensor, ws: torch.Tensor) -> None:
    """Speculative rejection sampling of one round: logits_t [x + 1][vocab], probs_d [x][vocab]
    (fp32, device), draft: the x drafts (a tensor or a device address)."""
    V = logits_t.shape[-1]
    d = draft if isinstance(draft, int) else ptr(draft)
    call("vc_spec_sample", V, ptr(logits_t), ptr(probs_d), d, x, C.byref(sampler), pos0, ptr(verified), ptr(ws),
         ws.numel(), stream_handle())


# ---------------------------------------------------------------- live kernel timing
def profile_enable(kinds=(VC_PROF_DRAFT_ATTN,)):
    """Time the given kernel classes (VC_PROF_*) from now on; an empty tuple stops."""
    mask = 0
    for k in kinds:
        mask |= 1 << k
    call("vc_profile_enable", mask)


def profile_read(kind: int = VC_PROF_DRAFT_ATTN) -> dict:
    """Totals of one kernel class since its last read (launches, event ms, algorithmic bytes
    and flops); clears that class's record."""
    st = ProfileStats()
    call("vc_profile_read", kind, C.byref(st))
    return {"launches": st.launches, "ms": st.total_ms, "bytes": st.bytes, "flops": st.flops,
            "aux_bytes": st.aux_bytes}


class PageableBuffer:
    """Ordinary (pageable) host memory for host rows beyond the pinned budget.  No copy
    engine ever reads or writes it: the engine moves its rows one layer at a time through
    pinned buffers with host memcpy (see Engine._offload_pageable / _stage_pageable).
    Never pass its address to a library call."""

    def __init__(self, nbytes: int):
        self.t = torch.empty(nbytes, dtype=torch.uint8)
        self.nbytes = nbytes

    def data_ptr(self) -> int:
        return self.t.data_ptr()

    def free(self):
        self.t = None


class HostBuffer:
    """Pinned host memory of an exact size (vc_host_alloc), freed with the object."""

    def __init__(self, nbytes: int):
        p = C.c_void_p()
        call("vc_host_alloc", nbytes, C.byref(p))
        self.ptr = p.value
        self.nbytes = nbytes
        self._view = None

    def data_ptr(self) -> int:
        return self.ptr

    def tensor(self) -> torch.Tensor:
        """A uint8 CPU tensor over the buffer (no copy; valid until free())."""
        if self._view is None:
            self._view = torch.frombuffer((C.c_uint8 * self.nbytes).from_address(self.ptr), dtype=torch.uint8)
        return self._view

    def free(self):
        self._view = None
        if self.ptr:
            call("vc_host_free", self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
