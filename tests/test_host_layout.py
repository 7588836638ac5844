"""Host-side logic of the C ABI that runs without a GPU: the section layout of a compressed
cache (VeriCache, section 3: a token-drop cache keeps K_keep, V_keep and the kept indices; a
quantized cache keeps per-group codes, scales and zero points and the unquantized remainder)
and the argument checks that reject unsupported settings before any device work."""
import pytest

import lossless_speculative_decoding_amd as vc
from lossless_speculative_decoding_amd._vc import VCError, VC_ERR_ARG, VC_ERR_UNSUPPORTED

L, HQ, HKV, D = 3, 8, 2, 128


def _sections(lay, names):
    return sorted((getattr(lay, n), n) for n in names)


def _check_disjoint(lay, sizes):
    """Sections start 256-byte aligned, in increasing order, and none overlaps the next
    (empty sections, e.g. no quantized group when T < group, take no space)."""
    secs = _sections(lay, [n for n in sizes if sizes[n] > 0])
    for (off, name), nxt in zip(secs, secs[1:] + [(lay.total, "end")]):
        assert off % 256 == 0, name
        assert off + sizes[name] <= nxt[0], (name, nxt[1])
    assert lay.total % 256 == 0


@pytest.mark.parametrize("T,keep,recent", [(1000, 250, 64), (64, 16, 64), (700, 900, 32), (129, 1, 0)])
def test_tokdrop_layout(T, keep, recent):
    d = vc.compress_desc(vc.VC_TOKDROP, L, HQ, HKV, D, T, vc.VC_BF16, keep_total=keep, keep_recent=recent)
    lay = vc.compress_layout(d)
    kk = min(T, max(keep, min(recent, T)))          # the recent window is always kept
    assert lay.n_main == kk and lay.n_resid == 0
    assert lay.n_host == T - kk                      # dropped rows live only on the host
    assert lay.n_tiles == -(-T // 64)
    row = D * 2
    sizes = {"k_main": L * HKV * kk * row, "v_main": L * HKV * kk * row, "idx": L * HKV * kk * 4,
             "keep_mask": L * HKV * lay.n_tiles * 8, "keep_cnt": L * HKV * lay.n_tiles * 4}
    _check_disjoint(lay, sizes)
    ob, _ = _size(d)
    assert ob == lay.total


@pytest.mark.parametrize("bits,group,T", [(2, 64, 1000), (3, 128, 1300), (4, 128, 127), (4, 64, 4096)])
def test_quant_layout(bits, group, T):
    d = vc.compress_desc(vc.VC_QUANT, L, HQ, HKV, D, T, vc.VC_BF16, bits=bits, group=group)
    lay = vc.compress_layout(d)
    tq = T // group * group
    assert lay.n_main == tq and lay.n_resid == T - tq
    assert lay.n_host == T                           # the host keeps the whole prompt
    ng = tq // group
    sizes = {"kc": L * HKV * tq * D * bits // 8, "vc": L * HKV * tq * D * bits // 8,
             "ks": L * HKV * ng * D * 2, "kz": L * HKV * ng * D * 2,
             "vs": L * HKV * tq * (D // group) * 2, "vz": L * HKV * tq * (D // group) * 2,
             "kr": L * HKV * (T - tq) * D * 2, "vr": L * HKV * (T - tq) * D * 2}
    _check_disjoint(lay, sizes)
    ob, _ = _size(d)
    assert ob == lay.total


def _size(d):
    import ctypes as C
    from lossless_speculative_decoding_amd._vc import call
    ob, wb = C.c_size_t(), C.c_size_t()
    call("vc_compress_size", C.byref(d), C.byref(ob), C.byref(wb))
    return ob.value, wb.value


@pytest.mark.parametrize("kw,code", [
    (dict(kind=vc.VC_QUANT, bits=5, group=128), VC_ERR_UNSUPPORTED),
    (dict(kind=vc.VC_QUANT, bits=1, group=128), VC_ERR_UNSUPPORTED),
    (dict(kind=vc.VC_QUANT, bits=4, group=32), VC_ERR_UNSUPPORTED),
    (dict(kind=vc.VC_QUANT, bits=4, group=128, head_dim=64), VC_ERR_UNSUPPORTED),
    (dict(kind=vc.VC_TOKDROP, seq_len=0), VC_ERR_ARG),
    (dict(kind=vc.VC_TOKDROP, src_cap=10), VC_ERR_ARG),
    (dict(kind=vc.VC_TOKDROP, keep_total=0), VC_ERR_ARG),
    (dict(kind=vc.VC_TOKDROP, n_q_heads=6, n_kv_heads=4), VC_ERR_ARG),
    (dict(kind=7), VC_ERR_ARG),
])
def test_layout_rejects_bad_settings(kw, code):
    args = dict(kind=vc.VC_TOKDROP, n_layers=L, n_q_heads=HQ, n_kv_heads=HKV, head_dim=D, seq_len=100,
                dtype=vc.VC_BF16, keep_total=25)
    args.update(kw)
    kind = args.pop("kind")
    d = vc.compress_desc(kind, args.pop("n_layers"), args.pop("n_q_heads"), args.pop("n_kv_heads"),
                         args.pop("head_dim"), args.pop("seq_len"), args.pop("dtype"), **args)
    with pytest.raises(VCError) as e:
        vc.compress_layout(d)
    assert e.value.code == code
