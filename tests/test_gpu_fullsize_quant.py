"""GPU parity at the kernel sizes of the two quantized-cache model workloads (one layer,
8B head shapes: 32 query heads over 8 KV heads of 128), on sampled (request, KV head)
slices the float64 oracle evaluates one by one.

- 2-bit, group 64: 4 requests x 131072 prompt rows; one batched draft step with a
  300-row exact tail per request; 41-row verification (x = 40) of every request.
- Mixed batch, 3-bit, group 128: 16 requests with the seeded log-uniform contexts of the
  mixed workload (most not a multiple of the group, so each keeps an exact residual) and
  ragged tails, one batched draft step over all 16; each sampled request verified with its
  own x + 1 rows (x from {16, 24, 32, 40}), one request per launch as in the model's
  verification.

K and V are N(0, 1) with 4 outlier channels per KV head scaled x10 (the single-layer
workload's recipe); each request has its own seed.  Compressed bytes of the sampled heads
are compared bit for bit, attention outputs per row within the bf16 tolerance."""
import numpy as np
import pytest

import synth
from gpu_helpers import TOL_BF16, dev_bf16, host_f64, log, need_gpu, row_rel_err, torch
from oracle import compress as OC
from oracle.model import attend

pytestmark = pytest.mark.gpu
HQ, HKV, D, G = 32, 8, 128, 4
f64 = lambda bits: synth.bf16_bits_to_f32(bits).astype(np.float64)


def _outl(seed):
    return np.stack([synth.outlier_channels_for(0, j, HKV, D, 4, seed) for j in range(HKV)]).astype(np.int32)


def _gen(rows, stream, seed, outl=None):
    from lossless_speculative_decoding_amd import synth_normal_heads
    t = torch.empty(1, HKV, rows, D, dtype=torch.bfloat16, device="cuda")
    o = torch.from_numpy(outl).cuda() if outl is not None else None
    synth_normal_heads(t, stream, o, 10.0, seed=seed)
    return t


def _host_head(stream, j, rows, seed, outl=None):
    return f64(synth.att_head(stream, 0, j, rows, HKV, D, None if outl is None else outl[j], 10.0, seed))


class Batch:
    """Per-request GPU inputs of one layer and their quantized blobs."""

    def __init__(self, ctx, bits, group, tail_rows, seed0):
        from lossless_speculative_decoding_amd import VC_BF16, VC_QUANT, compress_desc, vc_compress
        self.ctx, self.bits, self.group, self.seeds = ctx, bits, group, [seed0 + r for r in range(len(ctx))]
        self.tail_rows = tail_rows
        self.K, self.V, self.tK, self.tV, self.cds, self.blobs, self.outl = [], [], [], [], [], [], []
        for T, sd in zip(ctx, self.seeds):
            o = _outl(sd)
            K, V = _gen(T, synth.S_ATT_K, sd, o), _gen(T, synth.S_ATT_V, sd, o)
            d = compress_desc(VC_QUANT, 1, HQ, HKV, D, T, VC_BF16, bits=bits, group=group)
            self.blobs.append(vc_compress(d, K, V))
            self.cds.append(d)
            self.K.append(K[0])
            self.V.append(V[0])
            self.tK.append(_gen(tail_rows, synth.S_ATT_TK, sd)[0])
            self.tV.append(_gen(tail_rows, synth.S_ATT_TV, sd)[0])
            self.outl.append(o)
        torch.cuda.synchronize()

    def host(self, r, j):
        T, sd, o, nt = self.ctx[r], self.seeds[r], self.outl[r], self.tail_rows
        return dict(K=_host_head(synth.S_ATT_K, j, T, sd, o), V=_host_head(synth.S_ATT_V, j, T, sd, o),
                    tK=_host_head(synth.S_ATT_TK, j, nt, sd), tV=_host_head(synth.S_ATT_TV, j, nt, sd))

    def check_bytes(self, r, j, q):
        from lossless_speculative_decoding_amd import compress_layout
        lay = compress_layout(self.cds[r])
        b, g = self.bits, self.group
        Tq = self.ctx[r] // g * g
        ng, nb = Tq // g, Tq // 64
        sizes = dict(kc=Tq * D * b // 8, vc=nb * D * 8 * b, ks=ng * D * 2, kz=ng * D * 2, vs=Tq * (D // g) * 2,
                     vz=Tq * (D // g) * 2)
        want = dict(kc=OC.pack_bits(q.kcodes[0, 0], b).tobytes(),
                    vc=OC.pack_bits(q.vcodes[0, 0].reshape(nb, 64, D).transpose(0, 2, 1), b).tobytes(),
                    ks=q.ks[0, 0].astype("<f2").tobytes(), kz=q.kz[0, 0].astype("<f2").tobytes(),
                    vs=q.vs[0, 0].astype("<f2").tobytes(), vz=q.vz[0, 0].astype("<f2").tobytes())
        for name, n in sizes.items():
            off = getattr(lay, name) + j * n
            assert self.blobs[r][off:off + n].cpu().numpy().tobytes() == want[name], (r, j, name)

    def draft(self, n_tail):
        from lossless_speculative_decoding_amd import VC_BF16, VC_F32, vc_attn_draft
        from lossless_speculative_decoding_amd._vc import AttnDesc
        n = len(self.ctx)
        qd = np.stack([synth.att_queries(synth.S_ATT_QD, 0, 1, HQ, D, sd)[0] for sd in self.seeds])
        out = vc_attn_draft(AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_F32), self.blobs, self.cds, self.tK, self.tV,
                            list(n_tail), dev_bf16(qd))
        torch.cuda.synchronize()
        return qd, out

    def verify(self, r, n_rows):
        from lossless_speculative_decoding_amd import VC_BF16, VC_F32, vc_attn_verify
        from lossless_speculative_decoding_amd._vc import AttnDesc
        qv = synth.att_queries(synth.S_ATT_QV, 0, n_rows, HQ, D, self.seeds[r])
        out = vc_attn_verify(AttnDesc(HQ, HKV, D, VC_BF16, 0, VC_F32), dev_bf16(qv[None]), [self.K[r]], [self.V[r]],
                             [self.ctx[r]], [self.tK[r]], [self.tV[r]], n_rows)
        torch.cuda.synchronize()
        return qv, out[0]


def _check_request(bt, r, j, n_tail, qd, out_d, n_rows):
    h = bt.host(r, j)
    q = OC.Quantized(h["K"][None, None], h["V"][None, None], bt.bits, bt.group)
    bt.check_bytes(r, j, q)
    Kd = np.concatenate([q.rows_K()[0, 0], h["tK"][:n_tail]])
    Vd = np.concatenate([q.rows_V()[0, 0], h["tV"][:n_tail]])
    ref = np.stack([attend(f64(qd[r, j * G + g]), Kd, Vd) for g in range(G)])
    err_d = row_rel_err(host_f64(out_d[r, j * G:(j + 1) * G]), ref)
    qv, out_v = bt.verify(r, n_rows)
    err_v = 0.0
    for i in (0, n_rows // 2, n_rows - 1):
        K = np.concatenate([h["K"], h["tK"][:i + 1]])
        V = np.concatenate([h["V"], h["tV"][:i + 1]])
        ref = np.stack([attend(f64(qv[i, j * G + g]), K, V) for g in range(G)])
        err_v = max(err_v, row_rel_err(host_f64(out_v[i, j * G:(j + 1) * G]), ref))
    log(f"request {r} (T={bt.ctx[r]}, tail {n_tail}) head {j}: bytes exact; draft rel err {err_d:.2e}; "
        f"verify ({n_rows} rows) rel err {err_v:.2e}")
    assert err_d <= TOL_BF16 and err_v <= TOL_BF16


def test_q2g64_four_requests_131072():
    need_gpu()
    bt = Batch([131072] * 4, 2, 64, 300, seed0=40)
    qd, out = bt.draft([300] * 4)
    for r, j in [(0, 1), (3, 6)]:
        _check_request(bt, r, j, 300, qd, out, 41)


def test_q3g128_mixed_sixteen_requests():
    need_gpu()
    from synth.configs import llama8b_mixed
    w = llama8b_mixed()
    ctx, xs = list(w.ctx), list(w.x)
    tails = [1 + (37 * r) % 200 for r in range(len(ctx))]
    bt = Batch(ctx, 3, 128, 256, seed0=60)
    qd, out = bt.draft(tails)
    shortest, longest = int(np.argmin(ctx)), int(np.argmax(ctx))
    for r in (shortest, longest, 5):
        _check_request(bt, r, r % HKV, tails[r], qd, out, xs[r] + 1)
