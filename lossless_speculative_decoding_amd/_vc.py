"""ctypes binding of libvc.so (include/vc.h): structures and the C entry points.

Argument marshalling only -- every step of the path runs in the library's HIP
kernels.  Tensors are passed as raw device pointers (torch's data_ptr()),
streams as raw hipStream_t handles.  If the library is missing the import of
this module raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os

# PyTorch ships its own HIP runtime and asks for it as libamdhip64.so; libvc.so asks for
# libamdhip64.so.7.  Loaded in that order, the library binds to torch's runtime (same soname), so
# both share one runtime, its device and its streams.  Loaded the other way round the process
# would hold two runtimes, and the library's would see no device: torch is imported first.
import torch  # noqa: F401

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvc.so")

VC_OK, VC_ERR_ARG, VC_ERR_UNSUPPORTED, VC_ERR_CAPACITY, VC_ERR_HIP = 0, -1, -2, -3, -4
VC_F32, VC_BF16 = 0, 1
VC_TOKDROP, VC_QUANT = 1, 2
VC_SCORE_ATTN, VC_SCORE_KEYNORM = 0, 1
VC_MAX_BATCH = 16
(VC_PROF_DRAFT_ATTN, VC_PROF_VERIFY_ATTN, VC_PROF_GEMM_SKINNY, VC_PROF_GEMM_TILED,
 VC_PROF_PREFILL_ATTN) = range(5)


class VCError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


class ModelDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32), ("vocab", C.c_int32),
                ("dtype", C.c_int32), ("rope_theta", C.c_float), ("eps", C.c_float), ("max_pos", C.c_int32)]


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("embed", "lm_head", "norm_final", "norm_attn", "norm_ffn", "w_qkv", "w_o",
                                          "w_gu", "w_down")]


class CompressDesc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("kind", "bits", "group", "keep_total", "keep_recent", "obs_window",
                                         "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "seq_len", "dtype",
                                         "src_cap", "score")]


class CompressLayout(C.Structure):
    _fields_ = [("total", C.c_size_t), ("n_main", C.c_int32), ("n_resid", C.c_int32)] + \
               [(n, C.c_size_t) for n in ("k_main", "v_main", "idx", "kc", "vc", "ks", "kz", "vs", "vz", "kr", "vr",
                                          "keep_mask", "keep_cnt")] + \
               [("n_tiles", C.c_int32), ("n_host", C.c_int32)]


class Req(C.Structure):
    _fields_ = [("comp", C.c_void_p), ("cd", C.POINTER(CompressDesc)), ("tail_k", C.c_void_p), ("tail_v", C.c_void_p),
                ("tail_cap", C.c_int32), ("n_tail", C.c_int32), ("ctx_len", C.c_int32), ("draft_idx", C.c_int32),
                ("full_k_host", C.c_void_p), ("full_v_host", C.c_void_p), ("full_cap", C.c_int32),
                ("rows", C.c_void_p)]


class AttnDesc(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_q_heads", "n_kv_heads", "head_dim", "dtype", "split_len", "out_dtype")]


class ProfileStats(C.Structure):
    _fields_ = [("launches", C.c_int64), ("total_ms", C.c_double), ("bytes", C.c_double), ("flops", C.c_double),
                ("aux_bytes", C.c_double)]


class DebugStats(C.Structure):
    _fields_ = [("launches", C.c_int64), ("ranges", C.c_int64), ("violations", C.c_int64),
                ("pinned_bytes", C.c_double), ("pinned_peak", C.c_double)]


VC_DEBUG_OFF, VC_DEBUG_CHECK, VC_DEBUG_DRY = 0, 1, 2


class Sampler(C.Structure):
    _fields_ = [("temperature", C.c_float), ("seed", C.c_uint64), ("stream", C.c_uint64)]


VC_DRAW_DRAFT, VC_DRAW_ACCEPT, VC_DRAW_TARGET = 0, 1, 2


class AttnDraftReq(C.Structure):
    _fields_ = [("comp", C.c_void_p), ("cd", C.POINTER(CompressDesc)), ("tail_k", C.c_void_p),
                ("tail_v", C.c_void_p), ("tail_cap", C.c_int32), ("n_tail", C.c_int32)]


_P = C.c_void_p
_I = C.c_int32
_S = C.c_size_t
_SIGS = {
    "vc_last_error": (C.c_char_p, []),
    "vc_abi_version": (C.c_int32, []),
    "vc_model_create": (_I, [C.POINTER(ModelDesc), C.POINTER(Weights), _P, C.POINTER(_P)]),
    "vc_model_destroy": (_I, [_P]),
    "vc_ws_size": (_I, [_P, _I, _I, C.POINTER(_S)]),
    "vc_compress_layout_of": (_I, [C.POINTER(CompressDesc), C.POINTER(CompressLayout)]),
    "vc_compress_size": (_I, [C.POINTER(CompressDesc), C.POINTER(_S), C.POINTER(_S)]),
    "vc_compress": (_I, [C.POINTER(CompressDesc), _P, _P, _P, _P, _S, _P, _S, _P]),
    "vc_draft_step": (_I, [_P, C.POINTER(Req), _I, _P, _P, _S, _P]),
    "vc_draft_step_static": (_I, [_P, C.POINTER(Req), _I, _P, _P]),
    "vc_verify": (_I, [_P, C.POINTER(Req), _P, _P, _I, _P, _I, _P, _P, _P, _P, _I, _P, _S, _P]),
    "vc_verify_layered": (_I, [_P, C.POINTER(Req), _P, _P, _I, _P, _I, _P, _P, _P, _P, _I, _P, _S, _P, _P]),
    "vc_accept": (_I, [_P, C.POINTER(Req), _P, _I, _P, _P, _I, _P, _P]),
    "vc_commit": (_I, [_P, C.POINTER(Req), _I, _P, _P, _I, _P, _P]),
    "vc_stage": (_I, [_P, C.POINTER(Req), _P, _P, _I, _I, _I, _P]),
    "vc_prefill": (_I, [_P, _P, _I, _P, _P, _I, _P, _I, _P, _P, _I, _P, _S, _P]),
    "vc_sample": (_I, [_P, _I, _I, C.POINTER(Sampler), C.POINTER(C.c_int64), _I, _P, _P, _P]),
    "vc_draft_step_sampled": (_I, [_P, C.POINTER(Req), _I, C.POINTER(Sampler), C.POINTER(_P), _P, _P, _S, _P]),
    "vc_spec_ws_size": (_I, [_I, C.POINTER(_S)]),
    "vc_spec_sample": (_I, [_I, _P, _P, _P, _I, C.POINTER(Sampler), C.c_int64, _P, _P, _S, _P]),
    "vc_linear": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "vc_attn_ws_size": (_I, [C.POINTER(AttnDesc), _I, _I, _I, C.POINTER(_S)]),
    "vc_attn_draft": (_I, [C.POINTER(AttnDesc), C.POINTER(AttnDraftReq), _I, _P, _P, _P, _S, _P]),
    "vc_attn_verify": (_I, [C.POINTER(AttnDesc), _I, _P, C.POINTER(_P), C.POINTER(_P), _I, C.POINTER(_I),
                            C.POINTER(_P), C.POINTER(_P), _I, _I, _P, _P, _S, _P]),
    "vc_synth_xavier": (_I, [_P, _I, C.c_int64, C.c_uint32, C.c_uint32, C.c_int64, _I, _I, _P]),
    "vc_synth_normal_heads": (_I, [_P, _I, _I, _I, _I, C.c_uint32, C.c_uint32, _P, _I, C.c_float, _P]),
    "vc_synth_ids": (_I, [_P, C.c_int64, C.c_uint32, C.c_uint32, _I, _P]),
    "vc_synth_fill": (_I, [_P, _I, C.c_int64, C.c_float, _P]),
    "vc_profile_enable": (_I, [C.c_uint32]),
    "vc_host_alloc": (_I, [_S, C.POINTER(_P)]),
    "vc_host_free": (_I, [_P]),
    "vc_offload": (_I, [_P, C.POINTER(Req), _P, _P, _I, _I, _P]),
    "vc_offload_layers": (_I, [_P, C.POINTER(Req), _P, _P, _I, _I, _I, _I, _P]),
    "vc_profile_read": (_I, [_I, C.POINTER(ProfileStats)]),
    "vc_debug_mode": (_I, [_I]),
    "vc_debug_register": (_I, [_P, _S]),
    "vc_debug_forget": (_I, [_P]),
    "vc_debug_stats_read": (_I, [C.POINTER(DebugStats), _I]),
}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (or "
                      "python lossless_speculative_decoding_amd/csrc/build.py) first")
_lib = C.CDLL(LIB_PATH)
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def last_error() -> str:
    return _lib.vc_last_error().decode()


def call(name: str, *args) -> None:
    """Call a status-returning entry point; raise VCError on failure."""
    st = getattr(_lib, name)(*args)
    if st != VC_OK:
        raise VCError(name, st, last_error())


def raw(name: str):
    return getattr(_lib, name)


def exported_symbols():
    return list(_SIGS)
