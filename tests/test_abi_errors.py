"""Error behaviour of the C-ABI entry points, on the CPU.

Every entry point validates its arguments before it launches or copies anything, and returns the
status its declaration in include/vc.h names (VC_ERR_ARG for a bad argument, VC_ERR_CAPACITY for a
buffer or table too small, VC_ERR_UNSUPPORTED for a shape the kernels do not implement) with a
message from vc_last_error().  The calls run under the library's dry mode (no HIP call at all), on
a 1-layer bf16 model and a 2-bit request as the address-range tests build them; a valid call of
each entry point runs first, so the failure comes from the one argument changed."""
import ctypes as C

import pytest

from test_boundscheck import _dry_model, dry  # noqa: F401  (fixture)

ERR_ARG, ERR_UNSUPPORTED, ERR_CAPACITY = -1, -2, -3


def _fails(code, fn, *args, match=None):
    from lossless_speculative_decoding_amd._vc import VCError, call
    with pytest.raises(VCError, match=match) as e:
        call(fn, *args)
    assert e.value.code == code, str(e.value)


def test_model_create_rejects_shapes_it_does_not_implement(dry):  # noqa: F811
    from lossless_speculative_decoding_amd._vc import ModelDesc, Weights
    vc, m, eng, r = _dry_model()
    w = Weights(*[C.c_void_p(16) for _ in Weights._fields_])
    out = C.c_void_p()
    base = dict(n_layers=1, d_model=512, n_q_heads=4, n_kv_heads=1, head_dim=128, ffn=1024, vocab=1024,
                dtype=vc.VC_BF16, rope_theta=5e5, eps=1e-5, max_pos=64)
    for change, code in ((dict(head_dim=64), ERR_UNSUPPORTED),          # bf16 kernels are head_dim 128
                         (dict(n_q_heads=34, n_kv_heads=2), ERR_UNSUPPORTED),   # GQA group 17 > 16
                         (dict(n_q_heads=6, n_kv_heads=4), ERR_ARG),     # heads not a multiple
                         (dict(d_model=520), ERR_UNSUPPORTED),           # bf16 widths multiples of 128
                         (dict(max_pos=0), ERR_ARG)):
        d = ModelDesc(**{**base, **change})
        _fails(code, "vc_model_create", C.byref(d), C.byref(w), None, C.byref(out))
    d = ModelDesc(**base)
    _fails(ERR_ARG, "vc_model_create", C.byref(d), C.byref(Weights()), None, C.byref(out),
           match="null weight pointer")


def test_verify_rejects_bad_row_counts_and_small_buffers(dry):  # noqa: F811
    import torch
    vc, m, eng, r = _dry_model()
    ws = m.workspace(64, 4096, device="cpu")
    sk = torch.empty(1, 1, r.n_host, 128, dtype=torch.bfloat16)
    tok = torch.zeros(65, dtype=torch.int32)
    out = torch.zeros(65, dtype=torch.int32)
    vk = torch.empty(1, 1, 65, 128, dtype=torch.bfloat16)
    vc.debug_register(ws, sk, tok, out, vk)
    req = C.byref(r.req)
    args = lambda rows, vcap, scap=r.n_host: (m.h, req, sk.data_ptr(), sk.data_ptr(), scap, tok.data_ptr(), rows,
                                               out.data_ptr(), None, vk.data_ptr(), vk.data_ptr(), vcap,
                                               ws.data_ptr(), ws.numel(), None)
    from lossless_speculative_decoding_amd._vc import call
    call("vc_verify", *args(5, 65))                                   # valid
    _fails(ERR_ARG, "vc_verify", *args(0, 65), match="n_rows")
    _fails(ERR_ARG, "vc_verify", *args(65, 65), match="n_rows")
    _fails(ERR_CAPACITY, "vc_verify", *args(5, 4), match="vtail capacity")
    _fails(ERR_ARG, "vc_verify", *args(5, 65, r.n_host - 1), match="staged cache smaller")
    small = torch.empty(16, dtype=torch.uint8)
    vc.debug_register(small)
    a = list(args(5, 65))
    a[12], a[13] = small.data_ptr(), small.numel()
    _fails(ERR_CAPACITY, "vc_verify", *a, match="workspace")
    a = list(args(5, 65)) + [None]
    a[-2], a[-1] = None, None                                        # layer_ready, then the stream
    _fails(ERR_ARG, "vc_verify_layered", *a, match="null event array")


def test_accept_stage_offload_reject_bad_ranges(dry):  # noqa: F811
    import torch
    vc, m, eng, r = _dry_model()
    req = C.byref(r.req)
    res = torch.zeros(64, dtype=torch.int32)
    ver = torch.zeros(64, dtype=torch.int32)
    vk = torch.empty(1, 1, 8, 128, dtype=torch.bfloat16)
    vc.debug_register(res, ver, vk)
    acc = lambda x, vcap=8: (m.h, req, ver.data_ptr(), x, vk.data_ptr(), vk.data_ptr(), vcap, res.data_ptr(), None)
    from lossless_speculative_decoding_amd._vc import call
    call("vc_accept", *acc(4))                                        # valid
    _fails(ERR_ARG, "vc_accept", *acc(-1), match="draft length")
    _fails(ERR_ARG, "vc_accept", *acc(8), match="draft length")    # vtail must hold x + 1 rows
    r.req.n_tail = r.req.tail_cap - 2
    _fails(ERR_CAPACITY, "vc_accept", *acc(4), match="tail capacity")
    r.req.n_tail = 0
    slot = torch.empty(1, 1, r.n_host, 128, dtype=torch.bfloat16)
    vc.debug_register(slot)
    st = lambda l0, l1: (m.h, req, slot.data_ptr(), slot.data_ptr(), r.n_host, l0, l1, None)
    call("vc_stage", *st(0, 1))                                       # valid
    for l0, l1 in ((1, 0), (0, 2), (-1, 1)):
        _fails(ERR_ARG, "vc_stage", *st(l0, l1), match="layer range")
    kd = torch.empty(1, 1, 700, 128, dtype=torch.bfloat16)
    vc.debug_register(kd)
    off = lambda T, l0, l1: (m.h, req, kd.data_ptr(), kd.data_ptr(), 700, T, l0, l1, None)
    call("vc_offload_layers", *off(700, 0, 1))                       # valid
    _fails(ERR_ARG, "vc_offload_layers", *off(700, 0, 2), match="layer range")
    _fails(ERR_CAPACITY, "vc_offload_layers", *off(701, 0, 1), match="row counts")
    _fails(ERR_ARG, "vc_offload_layers", *off(600, 0, 1), match="rows given")


def test_draft_step_rejects_batches_past_the_limit(dry):  # noqa: F811
    vc, m, eng, r = _dry_model()
    from lossless_speculative_decoding_amd._vc import Req, call
    ws = m.workspace(1, 1024, device="cpu")
    vc.debug_register(ws)
    one = (Req * 1)(r.req)
    call("vc_draft_step", m.h, one, 1, None, ws.data_ptr(), ws.numel(), None)   # valid
    many = (Req * 17)(*([r.req] * 17))
    _fails(ERR_ARG, "vc_draft_step", m.h, many, 17, None, ws.data_ptr(), ws.numel(), None)
    _fails(ERR_ARG, "vc_draft_step", m.h, one, 0, None, ws.data_ptr(), ws.numel(), None)
