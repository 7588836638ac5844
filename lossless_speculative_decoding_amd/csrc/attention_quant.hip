// Draft-step decode attention over a per-group quantized KV cache (2/3/4-bit).
//
// One workgroup (256 threads) per (request, KV head, split of 64-key tiles).
// Per tile, all threads turn packed codes into exact small integers in fp16
// (magic-number trick: 0x6400 | c is 1024 + c, then subtract 1024) and stage
// them in LDS: K codes row-major (one row per key), V codes transposed (the
// packed layout is already per channel).  The quantization scale and zero are
// never applied to the codes; they are folded into the operands of the one
// computing wave instead:
//     q . k_t       = sum_d (q_d s_gd) c_td + sum_d q_d z_gd        (K: scale/zero per channel and token group)
//     sum_t p_t v_t = sum_t (p_t s_t) c_t  + sum_t p_t z_t          (V: scale/zero per token and channel group)
// so the MFMA operands are Q' = q*s, the codes, and P' = p*s (scaled by 2^10
// to stay out of the fp16 subnormal range).  Codes are centred (c - 2^(b-1),
// zero moves to z + 2^(b-1) s) so the folded sum does not cancel against a
// large zero term, and Q' and P' are each carried as an fp16 hi/lo pair (two
// MFMAs), which leaves about 22 significant bits in every score and weight.
//
// Within each group of 8 (4-bit) or 16 (2-bit) codes the conversion yields the
// codes in the order [0,4,1,5,2,6,3,7] (resp. [0,8,1,9,...,7,15]); LDS
// positions keep that order, for channels (K columns, mirrored in Q') and for
// keys (K rows and V^T columns, mirrored in the key index of each score).
#include "attention.h"

namespace vc {

namespace {

constexpr int D = 128;
constexpr int KS_PITCH = D + 8;
constexpr int VT_PITCH = ATT_KT + 8;
constexpr float P_SCALE = 1024.f;
constexpr float P_UNSCALE = 1.f / 1024.f;

// 0x6400 | c is the fp16 number 1024 + c; subtracting 1024 + 2^(b-1) leaves the centred code exactly
template <int BITS>
__device__ __forceinline__ uint32_t centre(uint32_t x) {
  constexpr float off = 1024.f + float(1 << (BITS - 1));
  return bitcast<uint32_t>(bitcast<f16x2>(x) - f16x2{(_Float16)off, (_Float16)off});
}

// position -> code index within a conversion group
template <int BITS>
__device__ __forceinline__ int perm_pos(int p) {
  if constexpr (BITS == 4) {
    const int k = p & 7;
    return (p & ~7) | ((k & 1) ? 4 + (k >> 1) : (k >> 1));
  } else if constexpr (BITS == 2) {
    const int k = p & 15;
    return (p & ~15) | ((k & 1) ? 8 + (k >> 1) : (k >> 1));
  } else {
    return p;
  }
}
// code index -> position (inverse of perm_pos)
template <int BITS>
__device__ __forceinline__ int inv_perm(int c) {
  if constexpr (BITS == 4) {
    const int k = c & 7;
    return (c & ~7) | ((k < 4) ? 2 * k : 2 * (k - 4) + 1);
  } else if constexpr (BITS == 2) {
    const int k = c & 15;
    return (c & ~15) | ((k < 8) ? 2 * k : 2 * (k - 8) + 1);
  } else {
    return c;
  }
}

template <int BITS>
struct Codes32 {
  uint32_t w[BITS];  // 32 * BITS bits
};

template <int BITS>
__device__ __forceinline__ Codes32<BITS> ld_codes(const uint8_t* src) {
  Codes32<BITS> c;
  if constexpr (BITS == 4) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(src);
    c.w[0] = x.x; c.w[1] = x.y; c.w[2] = x.z; c.w[3] = x.w;
  } else if constexpr (BITS == 2) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(src);
    c.w[0] = x.x; c.w[1] = x.y;
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(src);
    c.w[0] = p[0]; c.w[1] = p[1]; c.w[2] = p[2];
  }
  return c;
}

template <int BITS>
__device__ __forceinline__ void cvt_codes(const Codes32<BITS>& c, u32x4 out[4]) {
  constexpr uint32_t MAG = 0x64006400u;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const uint32_t x = c.w[w];
      out[w].x = centre<BITS>((x & 0x000F000Fu) | MAG);
      out[w].y = centre<BITS>(((x >> 4) & 0x000F000Fu) | MAG);
      out[w].z = centre<BITS>(((x >> 8) & 0x000F000Fu) | MAG);
      out[w].w = centre<BITS>(((x >> 12) & 0x000F000Fu) | MAG);
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int w = 0; w < 2; w++) {
      const uint32_t x = c.w[w];
      out[2 * w].x = centre<BITS>((x & 0x00030003u) | MAG);
      out[2 * w].y = centre<BITS>(((x >> 2) & 0x00030003u) | MAG);
      out[2 * w].z = centre<BITS>(((x >> 4) & 0x00030003u) | MAG);
      out[2 * w].w = centre<BITS>(((x >> 6) & 0x00030003u) | MAG);
      out[2 * w + 1].x = centre<BITS>(((x >> 8) & 0x00030003u) | MAG);
      out[2 * w + 1].y = centre<BITS>(((x >> 10) & 0x00030003u) | MAG);
      out[2 * w + 1].z = centre<BITS>(((x >> 12) & 0x00030003u) | MAG);
      out[2 * w + 1].w = centre<BITS>(((x >> 14) & 0x00030003u) | MAG);
    }
  } else {
    const uint64_t lo = uint64_t(c.w[0]) | (uint64_t(c.w[1]) << 32);
    const uint64_t hi = uint64_t(c.w[1]) | (uint64_t(c.w[2]) << 32);
    uint32_t r[16];
#pragma unroll
    for (int m = 0; m < 16; m++) {
      const int off = 6 * m;
      const uint32_t f = off < 32 ? uint32_t(lo >> off) : uint32_t(hi >> (off - 32));
      r[m] = centre<BITS>(((f & 7u) | ((f & 0x38u) << 13)) | MAG);
    }
#pragma unroll
    for (int q = 0; q < 4; q++) out[q] = u32x4{r[4 * q], r[4 * q + 1], r[4 * q + 2], r[4 * q + 3]};
  }
}

__device__ __forceinline__ float h2f(uint16_t h) { return float(bitcast<_Float16>(h)); }

template <int BITS>
__global__ __launch_bounds__(256) void attn_quant_kernel(const QuantArgs args) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[ATT_KT * KS_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VT_PITCH];
  __shared__ float vsc[ATT_KT][2];
  __shared__ float vzr[ATT_KT][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int z = blockIdx.z;
  if (z >= args.n_req) return;
  const QuantReq& R = args.r[z];
  const int Hkv = args.Hkv, G = args.G, Hq = args.Hq;
  const int j = blockIdx.x;
  const int s = blockIdx.y;
  if (s >= R.n_splits) return;
  const int Tq = R.m.tq;
  const int grp_sz = args.group;
  const int nh = D / grp_sz;      // V channel groups per token (1 or 2)
  const bool two_groups = nh == 2;
  const int ng = Tq / grp_sz;     // K token groups
  const int nblk = Tq / 64;
  const int key_lo = s * args.split_len;
  const int key_hi = min(key_lo + args.split_len, Tq);
  constexpr int RB = 4 * BITS;    // bytes of 32 codes

  const uint8_t* kc = R.m.kc + int64_t(j) * Tq * (D * BITS / 8);
  const uint8_t* vc = R.m.vc + int64_t(j) * nblk * D * (8 * BITS);
  const uint16_t* ks = R.m.ks + int64_t(j) * ng * D;
  const uint16_t* kz = R.m.kz + int64_t(j) * ng * D;
  const uint16_t* vs = R.m.vs + int64_t(j) * Tq * nh;
  const uint16_t* vz = R.m.vz + int64_t(j) * Tq * nh;

  const int grp = lane >> 4;
  const int qrow = lane & 15;
  const bool row_ok = qrow < G;
  const int hq = j * G + (row_ok ? qrow : 0);

  // wave 0: the query row of this lane, at the permuted channel positions it feeds
  float qv[4][8];
  if (wave == 0) {
    const uint16_t* qp = static_cast<const uint16_t*>(R.q) + int64_t(hq) * D;
#pragma unroll
    for (int c = 0; c < 4; c++) {
#pragma unroll
      for (int e = 0; e < 8; e++) qv[c][e] = row_ok ? bf2f(qp[perm_pos<BITS>(32 * c + 8 * grp + e)]) : 0.f;
    }
  }
  constexpr float C0 = float(1 << (BITS - 1));
  u32x4 qf[4], qlo[4];
  float kbias = 0.f;
  int cur_group = -1;
  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; dt++) oacc[dt] = f32x4{0, 0, 0, 0};
  float vb[2] = {0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;
  const float sl2 = args.scale_log2;

  for (int t0 = key_lo; t0 < key_hi; t0 += ATT_KT) {
    // ---- cooperative conversion of this tile
    Codes32<BITS> kcw, vcw;
    {
      const int key = tid >> 2, part = tid & 3;
      kcw = ld_codes<BITS>(kc + int64_t(t0 + key) * (D * BITS / 8) + part * RB);
      const int ch = tid >> 1, half = tid & 1;
      vcw = ld_codes<BITS>(vc + (int64_t(t0 / 64) * D + ch) * (8 * BITS) + half * RB);
    }
    float vsv[2] = {0.f, 0.f}, vzv[2] = {0.f, 0.f};
    if (tid < ATT_KT) {
      const int t = t0 + perm_pos<BITS>(tid);
      for (int h = 0; h < nh; h++) {
        vsv[h] = h2f(vs[int64_t(t) * nh + h]);
        vzv[h] = fmaf(vsv[h], float(1 << (BITS - 1)), h2f(vz[int64_t(t) * nh + h]));  // zero of the centred code
      }
    }
    __syncthreads();  // previous tile fully consumed
    {
      u32x4 kout[4], vout[4];
      cvt_codes<BITS>(kcw, kout);
      cvt_codes<BITS>(vcw, vout);
      const int key = tid >> 2, part = tid & 3;
      const int row = inv_perm<BITS>(key);
#pragma unroll
      for (int q = 0; q < 4; q++) *reinterpret_cast<u32x4*>(Ks + row * KS_PITCH + 32 * part + 8 * q) = kout[q];
      const int ch = tid >> 1, half = tid & 1;
#pragma unroll
      for (int q = 0; q < 4; q++) *reinterpret_cast<u32x4*>(Vt + ch * VT_PITCH + 32 * half + 8 * q) = vout[q];
      if (tid < ATT_KT) {
        vsc[tid][0] = vsv[0]; vsc[tid][1] = vsv[1];
        vzr[tid][0] = vzv[0]; vzr[tid][1] = vzv[1];
      }
    }
    __syncthreads();
    if (wave != 0) continue;

    // ---- Q' = q * s_g and the key bias of this token group
    const int g = t0 / grp_sz;
    if (g != cur_group) {
      cur_group = g;
      float b = 0.f;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        uint32_t w[4], wl[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; e2++) {
          const int ch0 = perm_pos<BITS>(32 * c + 8 * grp + 2 * e2);
          const int ch1 = perm_pos<BITS>(32 * c + 8 * grp + 2 * e2 + 1);
          const float s0 = h2f(ks[int64_t(g) * D + ch0]), s1 = h2f(ks[int64_t(g) * D + ch1]);
          const float z0 = h2f(kz[int64_t(g) * D + ch0]), z1 = h2f(kz[int64_t(g) * D + ch1]);
          const float a0 = qv[c][2 * e2], a1 = qv[c][2 * e2 + 1];
          b = fmaf(a0, fmaf(s0, C0, z0), b);
          b = fmaf(a1, fmaf(s1, C0, z1), b);
          const float p0 = a0 * s0, p1 = a1 * s1;
          const _Float16 h0 = (_Float16)p0, h1 = (_Float16)p1;
          w[e2] = bitcast<uint32_t>(f16x2{h0, h1});
          wl[e2] = bitcast<uint32_t>(f16x2{(_Float16)(p0 - float(h0)), (_Float16)(p1 - float(h1))});
        }
        qf[c] = u32x4{w[0], w[1], w[2], w[3]};
        qlo[c] = u32x4{wl[0], wl[1], wl[2], wl[3]};
      }
      b += shfl_xor(b, 16);
      b += shfl_xor(b, 32);
      kbias = b;
    }

    // ---- S^T = C_K Q'^T
    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
      sacc[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(Ks + (16 * kt + (lane & 15)) * KS_PITCH + 32 * c + 8 * grp);
        sacc[kt] = mfma_f16(ka, qf[c], sacc[kt]);
        sacc[kt] = mfma_f16(ka, qlo[c], sacc[kt]);
      }
    }
    float mx = NEG_INF;
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const float v = row_ok ? (sacc[kt][jj] + kbias) * sl2 : NEG_INF;
        sacc[kt][jj] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const bool none = (m_new == NEG_INF);
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const float p = none ? 0.f : __builtin_amdgcn_exp2f(sacc[kt][jj] - m_new);
        sacc[kt][jj] = p;
        rs += p;
      }
    }
    rs += shfl_xor(rs, 16);
    rs += shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) oacc[dt] *= alpha;
    vb[0] *= alpha;
    vb[1] *= alpha;

    // ---- O^T += C_V^T P'^T, one P' per channel group of V
#pragma unroll
    for (int kc2 = 0; kc2 < 2; kc2++) {
      float pv[8];
      int pos[8];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        pos[e] = 32 * kc2 + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
        pv[e] = sacc[2 * kc2 + (e >> 2)][e & 3] * P_SCALE;
      }
      // P' for each channel group of V (group 1 only exists when the V group is 64 channels)
      uint32_t w0[4], w1[4], l0[4], l1[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; e2++) {
        const int p0 = pos[2 * e2], p1 = pos[2 * e2 + 1];
        const float x0 = pv[2 * e2], x1 = pv[2 * e2 + 1];
        split_h2(x0 * vsc[p0][0], x1 * vsc[p1][0], w0[e2], l0[e2]);
        split_h2(x0 * vsc[p0][1], x1 * vsc[p1][1], w1[e2], l1[e2]);
        vb[0] = fmaf(x0, vzr[p0][0], vb[0]);
        vb[0] = fmaf(x1, vzr[p1][0], vb[0]);
        vb[1] = fmaf(x0, vzr[p0][1], vb[1]);
        vb[1] = fmaf(x1, vzr[p1][1], vb[1]);
      }
      const u32x4 pb0 = u32x4{w0[0], w0[1], w0[2], w0[3]};
      const u32x4 pb1 = two_groups ? u32x4{w1[0], w1[1], w1[2], w1[3]} : pb0;
      const u32x4 pl0 = u32x4{l0[0], l0[1], l0[2], l0[3]};
      const u32x4 pl1 = two_groups ? u32x4{l1[0], l1[1], l1[2], l1[3]} : pl0;
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
        const uint16_t* vrow = Vt + (16 * dt + (lane & 15)) * VT_PITCH + 32 * kc2 + 4 * grp;
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(vrow + 16);
        const u32x4 va = u32x4{v0.x, v0.y, v1.x, v1.y};
        oacc[dt] = mfma_f16(va, dt < 4 ? pb0 : pb1, oacc[dt]);
        oacc[dt] = mfma_f16(va, dt < 4 ? pl0 : pl1, oacc[dt]);
      }
    }
  }
  if (wave != 0) return;
  // the zero term of V is the same for every channel of a group: reduce over the key lanes
  float vbt[2];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    float b = vb[h];
    b += shfl_xor(b, 16);
    b += shfl_xor(b, 32);
    vbt[h] = b;
  }
  if (!row_ok) return;
  float* dst = R.part + (int64_t(hq) * R.s_total + s) * (D + 2);
  if (grp == 0) {
    dst[0] = m_run;
    dst[1] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 8; dt++) {
    const int h = two_groups ? (dt >> 2) : 0;
#pragma unroll
    for (int jj = 0; jj < 4; jj++) dst[2 + 16 * dt + 4 * grp + jj] = (oacc[dt][jj] + vbt[h]) * P_UNSCALE;
  }
}

}  // namespace

vc_status launch_attn_quant(const QuantArgs& a, hipStream_t s) {
  if (a.n_req <= 0 || a.max_splits <= 0) return VC_OK;
  VC_REQUIRE(a.group == 64 || a.group == 128, VC_ERR_UNSUPPORTED, "quant group must be 64 or 128");
  VC_REQUIRE(a.G <= 16, VC_ERR_UNSUPPORTED, "GQA group > 16");
  VC_REQUIRE(a.split_len % a.group == 0 || a.group % a.split_len == 0, VC_ERR_ARG, "split/group mismatch");
  dim3 grid(a.Hkv, a.max_splits, a.n_req);
  switch (a.bits) {
    case 2: hipLaunchKernelGGL(attn_quant_kernel<2>, grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(attn_quant_kernel<3>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(attn_quant_kernel<4>, grid, dim3(256), 0, s, a); break;
    default: VC_REQUIRE(false, VC_ERR_UNSUPPORTED, "bits must be 2, 3 or 4 (got %d)", a.bits);
  }
  VC_LAUNCH_CHECK();
  return VC_OK;
}

}  // namespace vc
