"""GPU parity of the compressor and the attention cores against the oracle
(single GQA layer with Llama-3-8B head shapes, at sizes that span several
splits, tiles and a ragged tail)."""
import numpy as np
import pytest

import synth
from gpu_helpers import TOL_BF16, bytes_of, dev_bf16, host_f64, log, need_gpu, row_rel_err, torch
from oracle import attention as OA
from oracle import compress as OC

pytestmark = pytest.mark.gpu
HQ, HKV, D = 32, 8, 128


def _head_bits(stream, b, T, outl=True):
    out = []
    for j in range(HKV):
        o = synth.outlier_channels_for(b, j, HKV, D) if outl else None
        out.append(synth.att_head(stream, b, j, T, HKV, D, o, 10.0 if outl else 1.0))
    return np.stack(out)[None]                     # [1][Hkv][T][D] uint16


def _f(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("bits,group,T", [(4, 128, 1000), (2, 64, 1000), (3, 128, 1300), (3, 64, 700),
                                          (4, 64, 128), (2, 128, 64 * 3)])
def test_quant_blob_bit_exact(bits, group, T):
    need_gpu()
    from lossless_speculative_decoding_amd import VC_BF16, VC_QUANT, compress_desc, vc_compress
    log(f"quant blob bits={bits} group={group} T={T}")
    L = 2
    kb = np.concatenate([_head_bits(synth.S_ATT_K, b, T) for b in range(L)])   # layers from two requests' draws
    vb = np.concatenate([_head_bits(synth.S_ATT_V, b, T) for b in range(L)])
    d = compress_desc(VC_QUANT, L, HQ, HKV, D, T, VC_BF16, bits=bits, group=group)
    blob = vc_compress(d, dev_bf16(kb), dev_bf16(vb))
    torch.cuda.synchronize()
    q = OC.Quantized(_f(kb), _f(vb), bits, group)
    want = OC.quant_blob(q, "bf16")
    got = bytes_of(blob)
    assert len(got) == len(want)
    if got != want:
        g = np.frombuffer(got, np.uint8)
        w = np.frombuffer(want, np.uint8)
        bad = np.nonzero(g != w)[0]
        pytest.fail(f"{len(bad)} bytes differ, first at {bad[:8]}")


def _quant_case(n_req, T, bits, group, n_tail):
    from lossless_speculative_decoding_amd import VC_BF16, VC_QUANT, compress_desc, vc_compress
    comps, cds, tks, tvs, refs = [], [], [], [], []
    q = np.zeros((n_req, HQ, D), dtype=np.uint16)
    for b in range(n_req):
        kb, vb = _head_bits(synth.S_ATT_K, b, T)[0], _head_bits(synth.S_ATT_V, b, T)[0]
        tk = _head_bits(synth.S_ATT_TK, b, n_tail, outl=False)[0]
        tv = _head_bits(synth.S_ATT_TV, b, n_tail, outl=False)[0]
        q[b] = synth.att_queries(synth.S_ATT_QD, b, 1, HQ, D)[0]
        d = compress_desc(VC_QUANT, 1, HQ, HKV, D, T, VC_BF16, bits=bits, group=group)
        cds.append(d)
        comps.append(vc_compress(d, dev_bf16(kb[None]), dev_bf16(vb[None])))
        tks.append(dev_bf16(tk))
        tvs.append(dev_bf16(tv))
        qq = OC.Quantized(_f(kb[None]), _f(vb[None]), bits, group)
        Kd, Vd = qq.rows_K()[0], qq.rows_V()[0]
        qf = _f(q[b])
        o = np.zeros((HQ, D))
        for j in range(HKV):
            K = np.concatenate([Kd[j], _f(tk[j])])
            V = np.concatenate([Vd[j], _f(tv[j])])
            for g in range(HQ // HKV):
                o[j * 4 + g] = OA.attend(qf[j * 4 + g], K, V)
        refs.append(o)
    return comps, cds, tks, tvs, q, np.stack(refs)


@pytest.mark.parametrize("bits,group,T,n_tail", [(4, 128, 2048 + 128, 5), (2, 64, 1984, 1), (3, 128, 1300, 33),
                                                 (4, 64, 3000, 64)])
def test_draft_attention_quant(bits, group, T, n_tail):
    need_gpu()
    from lossless_speculative_decoding_amd import VC_BF16, VC_F32, vc_attn_draft
    from lossless_speculative_decoding_amd._vc import AttnDesc
    log(f"draft attention quant bits={bits} group={group} T={T} tail={n_tail}")
    comps, cds, tks, tvs, q, ref = _quant_case(3, T, bits, group, n_tail)
    d = AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_F32)
    out = vc_attn_draft(d, comps, cds, tks, tvs, [n_tail] * 3, dev_bf16(q))
    torch.cuda.synchronize()
    err = row_rel_err(host_f64(out), ref)
    log("  rel err", err)
    assert err <= TOL_BF16


def _verify_case(n_req, ctxs, n_rows, cap):
    Kst, Vst, tks, tvs, refs = [], [], [], [], []
    q = np.zeros((n_req, n_rows, HQ, D), dtype=np.uint16)
    for b in range(n_req):
        T = ctxs[b]
        kb, vb = _head_bits(synth.S_ATT_K, b, T)[0], _head_bits(synth.S_ATT_V, b, T)[0]
        kpad = np.zeros((HKV, cap, D), np.uint16)
        vpad = np.zeros((HKV, cap, D), np.uint16)
        kpad[:, :T], vpad[:, :T] = kb, vb
        tk = _head_bits(synth.S_ATT_TK, b, n_rows, outl=False)[0]
        tv = _head_bits(synth.S_ATT_TV, b, n_rows, outl=False)[0]
        q[b] = synth.att_queries(synth.S_ATT_QV, b, n_rows, HQ, D)
        Kst.append(dev_bf16(kpad))
        Vst.append(dev_bf16(vpad))
        tks.append(dev_bf16(tk))
        tvs.append(dev_bf16(tv))
        qf = _f(q[b])
        o = np.zeros((n_rows, HQ, D))
        for i in range(n_rows):
            for j in range(HKV):
                K = np.concatenate([_f(kb[j]), _f(tk[j, : i + 1])])
                V = np.concatenate([_f(vb[j]), _f(tv[j, : i + 1])])
                for g in range(4):
                    o[i, j * 4 + g] = OA.attend(qf[i, j * 4 + g], K, V)
        refs.append(o)
    return Kst, Vst, tks, tvs, q, np.stack(refs)


@pytest.mark.parametrize("ctxs,n_rows", [((1500, 2100), 33), ((64, 1), 17), ((0, 130), 3), ((2048,), 1),
                                         ((700, 1250), 64),   # 256 query rows: two row groups, the most rows per call
                                         ((900,), 48)])       # 192 query rows: one full group of 12 row blocks
def test_verify_attention(ctxs, n_rows):
    need_gpu()
    from lossless_speculative_decoding_amd import VC_BF16, VC_F32, vc_attn_verify
    from lossless_speculative_decoding_amd._vc import AttnDesc
    log(f"verify attention ctxs={ctxs} rows={n_rows}")
    cap = max(max(ctxs), 1)
    Kst, Vst, tks, tvs, q, ref = _verify_case(len(ctxs), ctxs, n_rows, cap)
    d = AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_F32)
    out = vc_attn_verify(d, dev_bf16(q), Kst, Vst, list(ctxs), tks, tvs, n_rows, split_len=512)
    torch.cuda.synchronize()
    err = row_rel_err(host_f64(out), ref)
    log("  rel err", err)
    assert err <= TOL_BF16


def test_verify_row_invariance_bitwise():
    """Row i of a 33-row verify equals a 1-row verify at the same absolute
    position whose earlier tail rows sit in the staged cache instead."""
    need_gpu()
    from lossless_speculative_decoding_amd import VC_BF16, VC_F32, vc_attn_verify
    from lossless_speculative_decoding_amd._vc import AttnDesc
    ctx, n_rows = 1200, 33
    cap = ctx + n_rows
    Kst, Vst, tks, tvs, q, _ = _verify_case(1, (ctx,), 1, cap)        # staging only (reference unused)
    kb, vb = _head_bits(synth.S_ATT_K, 0, ctx)[0], _head_bits(synth.S_ATT_V, 0, ctx)[0]
    tk = _head_bits(synth.S_ATT_TK, 0, n_rows, outl=False)[0]
    tv = _head_bits(synth.S_ATT_TV, 0, n_rows, outl=False)[0]
    qb = synth.att_queries(synth.S_ATT_QV, 0, n_rows, HQ, D)
    d = AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_F32)
    kpad = np.zeros((HKV, cap, D), np.uint16)
    vpad = np.zeros((HKV, cap, D), np.uint16)
    kpad[:, :ctx], vpad[:, :ctx] = kb, vb
    many = vc_attn_verify(d, dev_bf16(qb[None]), [dev_bf16(kpad)], [dev_bf16(vpad)], [ctx], [dev_bf16(tk)],
                          [dev_bf16(tv)], n_rows)
    for i in (0, 1, 15, 16, 31, 32):
        k1, v1 = kpad.copy(), vpad.copy()
        k1[:, ctx:ctx + i], v1[:, ctx:ctx + i] = tk[:, :i], tv[:, :i]
        one = vc_attn_verify(d, dev_bf16(qb[None, i:i + 1]), [dev_bf16(k1)], [dev_bf16(v1)], [ctx + i],
                             [dev_bf16(tk[:, i:i + 1].copy())], [dev_bf16(tv[:, i:i + 1].copy())], 1)
        torch.cuda.synchronize()
        assert torch.equal(one[0, 0].view(torch.int16), many[0, i].view(torch.int16)), i


def test_tokdrop_blob_and_draft_attention():
    """Token-drop compression (scores, top-k, gather) and decode over kept rows + tail."""
    need_gpu()
    from lossless_speculative_decoding_amd import VC_BF16, VC_F32, VC_TOKDROP, compress_desc, vc_attn_draft, vc_compress
    from lossless_speculative_decoding_amd._vc import AttnDesc
    T, W, R, keep, n_tail = 1536, 32, 64, 384, 7
    kb, vb = _head_bits(synth.S_ATT_K, 0, T, outl=False)[0], _head_bits(synth.S_ATT_V, 0, T, outl=False)[0]
    qo = synth.att_queries(synth.S_ATT_QV, 1, W, HQ, D)                 # [W][Hq][D]
    d = compress_desc(VC_TOKDROP, 1, HQ, HKV, D, T, VC_BF16, keep_total=keep, keep_recent=R, obs_window=W)
    blob = vc_compress(d, dev_bf16(kb[None]), dev_bf16(vb[None]), dev_bf16(qo[None]))
    torch.cuda.synchronize()
    from lossless_speculative_decoding_amd import compress_layout
    lay = compress_layout(d)
    raw = blob.cpu().numpy()
    idx = raw[lay.idx: lay.idx + HKV * keep * 4].view(np.int32).reshape(HKV, keep)
    K, V = _f(kb), _f(vb)
    q_obs = _f(qo).transpose(1, 0, 2)[None]                            # oracle layout [L][Hq][W][D]
    widx, _, _, scores = OC.tokdrop(K[None], V[None], q_obs, keep, R, 4)
    for j in range(HKV):
        s = scores[0][j]
        got, want = set(idx[j].tolist()), set(widx[0, j].tolist())
        if got != want:
            # a differing element must sit at the top-k boundary within tolerance (flagged, not failed)
            kth = np.sort(s)[::-1][keep - R - 1]
            for t in got ^ want:
                assert abs(s[t] - kth) <= 1e-4 * kth, (j, t, s[t], kth)
        assert np.all(np.diff(idx[j]) > 0)
        kk = raw[lay.k_main:].view(np.uint16)[: HKV * keep * D].reshape(HKV, keep, D)
        assert np.array_equal(kk[j], kb[j, idx[j]])
    # decode over the kept rows + tail, against the oracle on the GPU's kept set
    tk = _head_bits(synth.S_ATT_TK, 0, n_tail, outl=False)[0]
    tv = _head_bits(synth.S_ATT_TV, 0, n_tail, outl=False)[0]
    qd = synth.att_queries(synth.S_ATT_QD, 0, 1, HQ, D)
    out = vc_attn_draft(AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_F32), [blob], [d], [dev_bf16(tk)], [dev_bf16(tv)], [n_tail],
                        dev_bf16(qd))
    torch.cuda.synchronize()
    ref = np.zeros((HQ, D))
    for j in range(HKV):
        Kj = np.concatenate([K[j, idx[j]], _f(tk[j])])
        Vj = np.concatenate([V[j, idx[j]], _f(tv[j])])
        for g in range(4):
            ref[j * 4 + g] = OA.attend(_f(qd[0, j * 4 + g]), Kj, Vj)
    err = row_rel_err(host_f64(out[0]), ref)
    log("  tokdrop draft rel err", err)
    assert err <= TOL_BF16


@pytest.mark.parametrize("reqs", [
    [(700, 200, 64, 70)],                                  # kept count off the 64-key grid, tail > 1 tile
    [(1536, 384, 64, 1), (900, 130, 32, 300), (2000, 777, 64, 65)],   # batch with mixed shapes
    [(640, 64, 64, 0), (512, 100, 64, 256)],               # kept = recent only, empty tail; 4-tile tail
    [(300 + 61 * b, 70 + 13 * b, 64, 9 * b) for b in range(16)],     # the largest batch one call takes
])
def test_draft_decode_ragged_batch(reqs):
    """One-row decode over (kept rows, tail) for a batch of requests of different sizes:
    kept counts off the tile grid, tails spanning tiles, an empty tail."""
    need_gpu()
    from lossless_speculative_decoding_amd import VC_BF16, VC_F32, VC_TOKDROP, compress_desc, compress_layout
    from lossless_speculative_decoding_amd import vc_attn_draft, vc_compress
    from lossless_speculative_decoding_amd._vc import AttnDesc
    W = 32
    blobs, cds, tks, tvs, ntl, host = [], [], [], [], [], []
    for b, (T, keep, R, n_tail) in enumerate(reqs):
        kb = _head_bits(synth.S_ATT_K, b, T, outl=False)[0]
        vb = _head_bits(synth.S_ATT_V, b, T, outl=False)[0]
        qo = synth.att_queries(synth.S_ATT_QV, b, W, HQ, D)
        d = compress_desc(VC_TOKDROP, 1, HQ, HKV, D, T, VC_BF16, keep_total=keep, keep_recent=R, obs_window=W)
        blob = vc_compress(d, dev_bf16(kb[None]), dev_bf16(vb[None]), dev_bf16(qo[None]))
        cap = max(n_tail, 1) + 5
        tk = np.zeros((HKV, cap, D), np.uint16)
        tv = np.zeros((HKV, cap, D), np.uint16)
        if n_tail:
            tk[:, :n_tail] = _head_bits(synth.S_ATT_TK, b, n_tail, outl=False)[0]
            tv[:, :n_tail] = _head_bits(synth.S_ATT_TV, b, n_tail, outl=False)[0]
        blobs.append(blob)
        cds.append(d)
        tks.append(dev_bf16(tk))
        tvs.append(dev_bf16(tv))
        ntl.append(n_tail)
        host.append((kb, vb, tk, tv, keep, n_tail))
    qd = synth.att_queries(synth.S_ATT_QD, 0, len(reqs), HQ, D)          # [B][Hq][D]
    out = vc_attn_draft(AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_F32), blobs, cds, tks, tvs, ntl, dev_bf16(qd))
    torch.cuda.synchronize()
    for b, (kb, vb, tk, tv, keep, n_tail) in enumerate(host):
        lay = compress_layout(cds[b])
        raw = blobs[b].cpu().numpy()
        idx = raw[lay.idx: lay.idx + HKV * keep * 4].view(np.int32).reshape(HKV, keep)
        ref = np.zeros((HQ, D))
        for j in range(HKV):
            Kj = np.concatenate([_f(kb[j, idx[j]]), _f(tk[j, :n_tail])])
            Vj = np.concatenate([_f(vb[j, idx[j]]), _f(tv[j, :n_tail])])
            for g in range(HQ // HKV):
                ref[j * (HQ // HKV) + g] = OA.attend(_f(qd[b, j * (HQ // HKV) + g]), Kj, Vj)
        err = row_rel_err(host_f64(out[b]), ref)
        log(f"  request {b} (T, keep, R, tail) = {reqs[b]}: rel err {err:.2e}")
        assert err <= TOL_BF16


def test_bf16_output_is_rounded_fp32_output():
    """The bf16 attention output is the fp32 result rounded to nearest even."""
    need_gpu()
    from lossless_speculative_decoding_amd import VC_BF16, VC_F32, vc_attn_verify
    from lossless_speculative_decoding_amd._vc import AttnDesc
    Kst, Vst, tks, tvs, q, _ = _verify_case(1, (700,), 5, 700)
    o32 = vc_attn_verify(AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_F32), dev_bf16(q), Kst, Vst, [700], tks, tvs, 5)
    o16 = vc_attn_verify(AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_BF16), dev_bf16(q), Kst, Vst, [700], tks, tvs, 5)
    torch.cuda.synchronize()
    want = synth.bf16_bits_from_f32(o32.cpu().numpy())
    assert np.array_equal(o16.view(torch.int16).cpu().numpy().view(np.uint16), want)


def test_profile_records_verify_and_draft_launches():
    """Live kernel timing (vc_profile_*): one record per launch group of the enabled class only,
    carrying the algorithmic bytes and flops the header defines for it."""
    need_gpu()
    import lossless_speculative_decoding_amd as vc
    from lossless_speculative_decoding_amd._vc import AttnDesc
    ctxs, rows, split = (1500, 2100), 33, 512
    cap = max(ctxs)  # one staged capacity for all requests
    Ks = [torch.randn(HKV, cap, D, device="cuda").to(torch.bfloat16) for _ in ctxs]
    Vs = [torch.randn(HKV, cap, D, device="cuda").to(torch.bfloat16) for _ in ctxs]
    tK = [torch.randn(HKV, rows, D, device="cuda").to(torch.bfloat16) for _ in ctxs]
    tV = [torch.randn(HKV, rows, D, device="cuda").to(torch.bfloat16) for _ in ctxs]
    q = torch.randn(len(ctxs), rows, HQ, D, device="cuda").to(torch.bfloat16)
    d = AttnDesc(HQ, HKV, D, vc.VC_BF16, 0, vc.VC_BF16)
    for k in range(5):
        vc.profile_read(k)
    vc.profile_enable((vc.VC_PROF_VERIFY_ATTN,))
    vc.vc_attn_verify(d, q, Ks, Vs, list(ctxs), tK, tV, rows, split_len=split)
    # a draft step while only verification is enabled: not recorded
    T, bits, group = 1000, 4, 128
    cd = vc.compress_desc(vc.VC_QUANT, 1, HQ, HKV, D, T, vc.VC_BF16, bits=bits, group=group)
    kq = torch.randn(1, HKV, T, D, device="cuda").to(torch.bfloat16)
    blob = vc.vc_compress(cd, kq, kq)
    qd = torch.randn(1, HQ, D, device="cuda").to(torch.bfloat16)
    vc.vc_attn_draft(d, [blob], [cd], [tK[0]], [tV[0]], [3], qd)
    vc.profile_enable((vc.VC_PROF_DRAFT_ATTN,))
    vc.vc_attn_draft(d, [blob], [cd], [tK[0]], [tV[0]], [3], qd)
    vc.profile_enable(())
    torch.cuda.synchronize()
    st = vc.profile_read(vc.VC_PROF_VERIFY_ATTN)
    want_b = want_f = want_a = 0.0
    for c in ctxs:
        S = -(-(c + rows) // split)
        want_b += HKV * (c + rows) * D * 2 * 2 + rows * HQ * D * 2
        want_a += rows * HQ * S * (D + 2) * 4          # the launch's own split partials, reported apart
        want_f += 4 * D * HQ * (rows * c + rows * (rows + 1) / 2)
    assert st["launches"] == 1 and st["ms"] > 0
    assert st["bytes"] == want_b and st["flops"] == want_f and st["aux_bytes"] == want_a
    sd = vc.profile_read(vc.VC_PROF_DRAFT_ATTN)
    Tq = T // group * group
    n_resid, n_tail = T - Tq, 3
    # quantized splits of 16 groups (2048 keys at group 128, G = 4); the exact rows are one slot
    s_quant, s_exact = -(-Tq // 2048), 1
    want = (HKV * (2 * Tq * D * bits / 8 + 2 * (Tq // group) * D * 2 + 2 * Tq * (D // group) * 2)
            + HKV * (n_resid + n_tail) * D * 2 * 2 + HQ * D * 2)
    assert sd["launches"] == 1 and sd["ms"] > 0
    assert sd["bytes"] == want, (sd["bytes"], want)
    assert sd["aux_bytes"] == HQ * (s_quant + s_exact) * (D + 2) * 4
    assert sd["flops"] == 4 * D * HQ * (T + n_tail)
    for k in (vc.VC_PROF_GEMM_SKINNY, vc.VC_PROF_GEMM_TILED, vc.VC_PROF_PREFILL_ATTN):
        assert vc.profile_read(k)["launches"] == 0


def test_v_beyond_fp16_range_is_non_finite_not_wrong():
    """A V element beyond fp16's range (the documented bound |v| <= 65504 of
    the verification kernel, which runs P.V on fp16) makes exactly the output
    channels it feeds non-finite there (staged row), and every other output
    still matches the oracle.  The draft kernel keeps V in bf16, so the same
    element in its tail row gives finite outputs that all match the oracle."""
    need_gpu()
    from lossless_speculative_decoding_amd import VC_BF16, VC_F32, VC_TOKDROP, compress_desc, compress_layout
    from lossless_speculative_decoding_amd import vc_attn_draft, vc_attn_verify, vc_compress
    from lossless_speculative_decoding_amd._vc import AttnDesc
    big = np.uint16(0x47C3)                                     # bf16 99840
    ctx, n_rows, ch, key = 300, 3, 7, 5
    Kst, Vst, tks, tvs, q, ref = _verify_case(1, (ctx,), n_rows, ctx)
    vb = Vst[0].cpu().view(torch.int16).numpy().view(np.uint16).copy()
    vb[0, key, ch] = big
    out = vc_attn_verify(AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_F32), dev_bf16(q), Kst, [dev_bf16(vb)], [ctx], tks, tvs,
                         n_rows, split_len=256)
    torch.cuda.synchronize()
    o = host_f64(out)[0]                                        # [rows][Hq][D]
    bad = ~np.isfinite(o)
    assert bad[:, 0:4, ch].all()                                # the four query heads of KV head 0, channel ch
    bad[:, 0:4, ch] = False
    assert not bad.any()
    keep = np.ones(o.shape, bool)
    keep[:, 0:4, ch] = False
    assert np.abs(o - ref[0])[keep].max() <= TOL_BF16 * np.abs(ref[0]).max()
    # draft kernel: the large element sits in the bf16 tail of KV head 3
    T, W, R, kt, n_tail = 640, 32, 64, 192, 5
    kb, vb2 = _head_bits(synth.S_ATT_K, 0, T, outl=False)[0], _head_bits(synth.S_ATT_V, 0, T, outl=False)[0]
    qo = synth.att_queries(synth.S_ATT_QV, 1, W, HQ, D)
    d = compress_desc(VC_TOKDROP, 1, HQ, HKV, D, T, VC_BF16, keep_total=kt, keep_recent=R, obs_window=W)
    blob = vc_compress(d, dev_bf16(kb[None]), dev_bf16(vb2[None]), dev_bf16(qo[None]))
    tk = _head_bits(synth.S_ATT_TK, 0, n_tail, outl=False)[0]
    tv = _head_bits(synth.S_ATT_TV, 0, n_tail, outl=False)[0]
    tv[3, 2, ch] = big
    qd = synth.att_queries(synth.S_ATT_QD, 0, 1, HQ, D)
    out = vc_attn_draft(AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_F32), [blob], [d], [dev_bf16(tk)], [dev_bf16(tv)],
                        [n_tail], dev_bf16(qd))
    torch.cuda.synchronize()
    o = host_f64(out[0])
    assert np.isfinite(o).all()
    raw = blob.cpu().numpy()
    idx = raw[compress_layout(d).idx: compress_layout(d).idx + HKV * kt * 4].view(np.int32).reshape(HKV, kt)
    for j in (0, 3):
        Kj = np.concatenate([_f(kb[j, idx[j]]), _f(tk[j])])
        Vj = np.concatenate([_f(vb2[j, idx[j]]), _f(tv[j])])
        for g in range(4):
            r = OA.attend(_f(qd[0, j * 4 + g]), Kj, Vj)
            assert np.abs(o[j * 4 + g] - r).max() <= TOL_BF16 * np.abs(r).max()
