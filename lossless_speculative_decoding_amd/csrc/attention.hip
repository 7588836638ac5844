// Attention kernels: split-K partials over bf16/fp32 key segments, the
// fixed-order combine, and (in attention_quant.hip) the quantized-cache decode.
//
// bf16 kernel (head_dim 128), one workgroup = 4 waves = (request, KV head,
// 64-row block, split).  Per 64-key tile the whole workgroup stages K (row
// major) and V (transposed, keys contiguous per channel) in LDS; each wave
// that owns 16 query rows then computes
//     S^T = K Q^T      (16x16x32 bf16 MFMA, A = K rows, B = Q^T fragments)
//     online softmax per query row (rows live in lanes l % 16)
//     O^T += V^T P^T   (A = V^T from LDS, B = P^T straight from the S^T registers)
// The S^T output layout puts row q = l%16 with keys 4*(l/16)+j of each 16-key
// sub-tile in lane l, which is exactly the B-operand layout P^T needs once the
// 32 keys of a chunk are enumerated as {4g..4g+3, 16+4g..16+4g+3}; V^T is read
// in that same key order, so no cross-lane shuffle of P is needed.
// The P.V product runs in fp16: V is converted from bf16 while it is staged
// (exact for |v| in [2^-14, 65504]) and P * 2^10 (P <= 1) is carried as an fp16
// hi/lo pair (hi = fp16(P), lo = fp16(P - hi), two MFMAs), which keeps about
// 22 significant bits of every weight; QK^T is bf16 x bf16 with exact products.
// Attention outputs then agree with a float64 evaluation to ~1e-6, so the
// bf16 rounding of the output (and of everything downstream) almost never
// lands on the other side of a rounding boundary than the exact value does.
#include "attention.h"

namespace vc {

namespace {

constexpr int D128 = 128;
constexpr int KS_PITCH = D128 + 8;     // bf16 per K row in LDS (pad breaks bank aliasing)
constexpr int VT_PITCH = ATT_KT + 8;   // fp16 per V^T row in LDS
constexpr float P_SCALE = 1024.f;      // P is rounded to fp16 as P * 2^10
constexpr float P_UNSCALE = 1.f / 1024.f;

struct TileRegs {
  u32x4 k[4];
  u32x4 v[4];
};

// Base pointers of tile [t0, t0 + 64) when it lies inside one plain segment (no segment
// boundary, not the kept/staged split of the prompt, not past the last key).
__device__ __forceinline__ bool tile_plain(const AttnReq& R, int j, int t0, int n_keys, const uint16_t*& kb,
                                           const uint16_t*& vb) {
  if (t0 + ATT_KT > n_keys) return false;
  const int an = R.a.n, bn = R.b.n;
  const KVSeg* sg;
  int off;
  if (t0 + ATT_KT <= an) {
    if (R.mix.mask != nullptr) return false;
    sg = &R.a;
    off = t0;
  } else if (t0 >= an && t0 + ATT_KT <= an + bn) {
    sg = &R.b;
    off = t0 - an;
  } else if (t0 >= an + bn) {
    sg = &R.c;
    off = t0 - an - bn;
  } else {
    return false;
  }
  const int64_t o = j * sg->hstride + int64_t(off) * D128;
  kb = static_cast<const uint16_t*>(sg->k) + o;
  vb = static_cast<const uint16_t*>(sg->v) + o;
  return true;
}

// K: thread (kr = tid/16, ch = tid%16) loads 16-byte chunk ch of keys kr + 16e (e = 0..3):
//    sixteen consecutive lanes move one whole 256-byte row (coalesced in HBM, and their LDS
//    stores cover all banks once).
// V: thread (dc = tid/16, kg = tid%16) loads channels 8dc..8dc+7 of keys 4kg..4kg+3.
__device__ __forceinline__ void load_tile_bf16(TileRegs& r, const AttnReq& R, int j, int t0, int n_keys, int tid) {
  const int kr = tid >> 4, ch = tid & 15, dc = tid >> 4, kg = tid & 15;
  const uint16_t* kb;
  const uint16_t* vb;
  if (tile_plain(R, j, t0, n_keys, kb, vb)) {  // uniform across the workgroup
#pragma unroll
    for (int e = 0; e < 4; e++) r.k[e] = *reinterpret_cast<const u32x4*>(kb + (kr + 16 * e) * D128 + 8 * ch);
#pragma unroll
    for (int e = 0; e < 4; e++) r.v[e] = *reinterpret_cast<const u32x4*>(vb + (4 * kg + e) * D128 + 8 * dc);
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int t = t0 + kr + 16 * e;
    r.k[e] = t < n_keys ? *reinterpret_cast<const u32x4*>(key_row<uint16_t, D128>(R, j, t, false) + 8 * ch)
                        : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int e = 0; e < 4; e++) {
    const int t = t0 + 4 * kg + e;
    r.v[e] = t < n_keys ? *reinterpret_cast<const u32x4*>(key_row<uint16_t, D128>(R, j, t, true) + 8 * dc)
                        : u32x4{0, 0, 0, 0};
  }
}

// V^T in LDS: row d holds the tile's 64 keys in fp16, key 32kc + 16h + 4g + jj at slot
// 32kc + 8g + 4h + jj, so the eight keys of one lane's P^T fragment are contiguous.
__device__ __forceinline__ void store_tile_bf16(const TileRegs& r, uint16_t* Ks, uint16_t* Vt, int tid) {
  const int kr = tid >> 4, ch = tid & 15, dc = tid >> 4, kg = tid & 15;
#pragma unroll
  for (int e = 0; e < 4; e++) *reinterpret_cast<u32x4*>(Ks + (kr + 16 * e) * KS_PITCH + 8 * ch) = r.k[e];
  const int slot = 32 * (kg >> 3) + 8 * (kg & 3) + 4 * ((kg >> 2) & 1);  // keys 4kg .. 4kg + 3
#pragma unroll
  for (int c = 0; c < 8; c++) {
    const int w = c >> 1;
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; e++) x[e] = (c & 1) ? hi_bf(r.v[e][w]) : lo_bf(r.v[e][w]);
    u32x2 out;
    out.x = bitcast<uint32_t>(f16x2{(_Float16)x[0], (_Float16)x[1]});
    out.y = bitcast<uint32_t>(f16x2{(_Float16)x[2], (_Float16)x[3]});
    *reinterpret_cast<u32x2*>(Vt + (8 * dc + c) * VT_PITCH + slot) = out;
  }
}

// Rows kernel (verification, prefill, observation scores): workgroup = 4 waves =
// (request, KV head, group of up to 64 * RPW query rows, split); wave w owns the 16-row
// blocks w, w + 4, ... (RPW of them), so every K/V tile staged in LDS serves all the
// rows of the group: a 33-row verification of 4 GQA heads (132 query rows) reads the
// keys once.  Each row's arithmetic is the same whatever block or group holds it.
template <int RPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_rows_bf16_kernel(
    const AttnArgs args) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[ATT_KT * KS_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D128 * VT_PITCH];
  constexpr int GROUP_ROWS = ATT_RB * RPW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int z = blockIdx.z;
  if (z >= args.n_req) return;
  const AttnReq& R = args.r[z];
  const int Hkv = args.Hkv, G = args.G, Hq = args.Hq;
  const int j = blockIdx.x % Hkv, rg = blockIdx.x / Hkv;
  const int s = blockIdx.y;
  const int n_qrows = R.n_rows * G;
  const int qr0 = rg * GROUP_ROWS;
  if (qr0 >= n_qrows || s >= R.n_splits) return;  // uniform across the workgroup

  const int n_keys = R.a.n + R.b.n + R.c.n;
  const int key_lo = s * args.split_len;
  const int i_max = (min(qr0 + GROUP_ROWS, n_qrows) - 1) / G;
  const int key_hi = min(min(key_lo + args.split_len, n_keys), R.lim0 + i_max + 1);
  const int grp = lane >> 4;

  // per row block of this wave: the lane's query row, its query fragments and state
  bool row_ok[RPW], blk_on[RPW];
  int qi[RPW], hq[RPW], lim[RPW];
  u32x4 qf[RPW][4];
  f32x4 oacc[RPW][8];
  float m_run[RPW], l_run[RPW];
#pragma unroll
  for (int b = 0; b < RPW; b++) {
    const int blk0 = qr0 + 16 * (wave + 4 * b);
    const int qr = blk0 + (lane & 15);
    blk_on[b] = blk0 < n_qrows;
    row_ok[b] = qr < n_qrows;
    qi[b] = row_ok[b] ? qr / G : 0;
    hq[b] = j * G + (row_ok[b] ? qr % G : 0);
    lim[b] = R.lim0 + qi[b];
    const uint16_t* qp = static_cast<const uint16_t*>(R.q) + (int64_t(qi[b]) * Hq + hq[b]) * D128;
#pragma unroll
    for (int c = 0; c < 4; c++)
      qf[b][c] = row_ok[b] ? *reinterpret_cast<const u32x4*>(qp + 32 * c + 8 * grp) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int dt = 0; dt < 8; dt++) oacc[b][dt] = f32x4{0, 0, 0, 0};
    m_run[b] = NEG_INF;
    l_run[b] = 0.f;
  }
  const float sl2 = args.scale_log2;

  TileRegs regs;
  if (key_lo < key_hi) load_tile_bf16(regs, R, j, key_lo, n_keys, tid);
  for (int t0 = key_lo; t0 < key_hi; t0 += ATT_KT) {
    __syncthreads();
    store_tile_bf16(regs, Ks, Vt, tid);
    __syncthreads();
    if (t0 + ATT_KT < key_hi) load_tile_bf16(regs, R, j, t0 + ATT_KT, n_keys, tid);

#pragma unroll
    for (int b = 0; b < RPW; b++) {
      if (!blk_on[b]) continue;  // uniform across the wave
      // ---- S^T = K Q^T over 4 sub-tiles of 16 keys
      f32x4 sacc[4];
#pragma unroll
      for (int kt = 0; kt < 4; kt++) {
        sacc[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(Ks + (16 * kt + (lane & 15)) * KS_PITCH + 32 * c + 8 * grp);
          sacc[kt] = mfma_bf16(ka, qf[b][c], sacc[kt]);
        }
      }
      // ---- scale, mask, online softmax (row q = lane % 16)
      float mx = NEG_INF;
#pragma unroll
      for (int kt = 0; kt < 4; kt++) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int t = t0 + 16 * kt + 4 * grp + jj;
          const bool vis = row_ok[b] && t < n_keys && t <= lim[b];
          const float v = vis ? sacc[kt][jj] * sl2 : NEG_INF;
          sacc[kt][jj] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[b], mx);
      const bool none = (m_new == NEG_INF);
      const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run[b] - m_new);
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
      l_run[b] = l_run[b] * alpha + rs;
      m_run[b] = m_new;
      if (__any(alpha != 1.f)) {  // x * 1 == x: skip the rescale when no running max moved
#pragma unroll
        for (int dt = 0; dt < 8; dt++) oacc[b][dt] *= alpha;
      }

      // ---- O^T += V^T P^T over 2 chunks of 32 keys
#pragma unroll
      for (int kc = 0; kc < 2; kc++) {
        uint32_t h[4], lw[4];
        split_h2(sacc[2 * kc][0] * P_SCALE, sacc[2 * kc][1] * P_SCALE, h[0], lw[0]);
        split_h2(sacc[2 * kc][2] * P_SCALE, sacc[2 * kc][3] * P_SCALE, h[1], lw[1]);
        split_h2(sacc[2 * kc + 1][0] * P_SCALE, sacc[2 * kc + 1][1] * P_SCALE, h[2], lw[2]);
        split_h2(sacc[2 * kc + 1][2] * P_SCALE, sacc[2 * kc + 1][3] * P_SCALE, h[3], lw[3]);
        const u32x4 pb = u32x4{h[0], h[1], h[2], h[3]};
        const u32x4 pl = u32x4{lw[0], lw[1], lw[2], lw[3]};
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
          const u32x4 va = *reinterpret_cast<const u32x4*>(Vt + (16 * dt + (lane & 15)) * VT_PITCH + 32 * kc + 8 * grp);
          oacc[b][dt] = mfma_f16(va, pb, oacc[b][dt]);
          oacc[b][dt] = mfma_f16(va, pl, oacc[b][dt]);
        }
      }
    }
  }

  // ---- partial (m, l, o) of this lane's rows; lane holds o[16dt + 4g + jj]
#pragma unroll
  for (int b = 0; b < RPW; b++) {
    if (!blk_on[b] || !row_ok[b]) continue;
    float* dst = R.part + ((int64_t(qi[b]) * Hq + hq[b]) * R.s_total + (R.s_off + s)) * (D128 + 2);
    if (grp == 0) {
      dst[0] = m_run[b];
      dst[1] = l_run[b];
    }
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) dst[2 + 16 * dt + 4 * grp + jj] = oacc[b][dt][jj] * P_UNSCALE;
    }
  }
}

// ---------------------------------------------------------------- bf16 decode, one query row
// Draft steps attend with a single query row per request, so a 64-row block would leave
// three of four waves idle.  Here one workgroup = 4 waves = (request, KV head, split) and
// wave w streams the 64-key tiles w, w + 4, w + 8, ... of the split on its own, with its own
// online softmax; the four states are merged in wave order at the end (fixed order, so the
// result does not depend on timing).  The G query heads of the KV head are the 16 MFMA
// columns.  K goes from HBM straight into A fragments (lane l: key l%16 of a 16-key group,
// channels 8(l/16)..+8 of a 32-channel chunk); V is converted to fp16 and transposed
// through a 16 KB LDS tile per wave.  A wave issues the next tile's loads as soon as the
// current tile's registers are consumed, so its softmax and P.V overlap the next fetch;
// KV loads are non-temporal (every byte is read once).
// V^T tile layout: row d (channel) holds 64 fp16 slots; key 32kc + 16h + 4g + jj of the tile
// sits in slot 32kc + 8g + 4h + jj, so the eight keys one lane's P^T fragment covers are
// contiguous; 16-byte groups are XOR-swizzled by dec_sw(d) to spread the fragment reads of
// 16 consecutive channels over all banks.
constexpr int DEC_WAVES = 4;
constexpr int DEC_TILE = D128 * ATT_KT;  // fp16 per wave LDS tile
constexpr int DEC_RED = D128 + 4;        // floats per head in the merge buffer

struct DecK {
  u32x4 k[4][4];  // [16-key group kt][32-channel chunk c]
};
struct DecV {
  u32x4 v[4][4];  // [16-key group a][key 4g + jj within it: jj]
};

__device__ __forceinline__ int dec_sw(int d) { return (d ^ (d >> 3)) & 7; }

// The decode kernel numbers keys per tile-aligned segment: segment a occupies logical
// keys [0, a_al) with a_al = a.n rounded up to 64 (keys a.n .. a_al - 1 are invisible),
// segment b follows at a_al.  Every 64-key tile then lies in one segment and is fetched
// through a buffer resource whose range ends at the segment's last row, so rows past it
// read as zero without per-row branches.
struct DecOff {
  int k[4];  // byte offset of this lane's K fragment row in 16-key group kt
  int v[4];  // byte offset of this lane's V row (jj = 0) in 16-key group q
};

__device__ __forceinline__ void dec_load(DecK& K, DecV& V, const KVSeg& a, const KVSeg& b, int a_al, int j, int t0,
                                         const DecOff& off) {
  const bool in_a = t0 < a_al;
  const KVSeg& sg = in_a ? a : b;
  const int row0 = in_a ? t0 : t0 - a_al;
  const int64_t base = j * sg.hstride + int64_t(row0) * D128;
  const int bytes = max(sg.n - row0, 0) * (D128 * 2);
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(sg.k) + base), 0, bytes, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(static_cast<const uint16_t*>(sg.v) + base), 0, bytes, BUF_DWORD3);
#pragma unroll
  for (int kt = 0; kt < 4; kt++) {
#pragma unroll
    for (int c = 0; c < 4; c++) K.k[kt][c] = ld_buf_nt(rk, off.k[kt] + 64 * c);
  }
#pragma unroll
  for (int q = 0; q < 4; q++) {
#pragma unroll
    for (int jj = 0; jj < 4; jj++) V.v[q][jj] = ld_buf_nt(rv, off.v[q] + jj * D128 * 2);
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_decode_bf16_kernel(const AttnArgs args) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[DEC_WAVES * DEC_TILE];
  // the wave index is uniform per wave; readfirstlane lets the compiler keep the tile
  // addresses (and the buffer resources built from them) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int z = blockIdx.z;
  if (z >= args.n_req) return;
  const AttnReq& R = args.r[z];
  const int G = args.G, Hq = args.Hq;
  const int j = blockIdx.x, s = blockIdx.y;
  if (s >= R.n_splits) return;  // uniform across the workgroup
  const int a_n = R.a.n, a_al = (a_n + ATT_KT - 1) & ~(ATT_KT - 1);
  const int key_lo = s * args.split_len;
  const int key_hi = min(key_lo + args.split_len, a_al + R.b.n);
  const int r16 = lane & 15, g = lane >> 4;
  const bool head_ok = r16 < G;
  uint16_t* Vt = lds + wave * DEC_TILE;
  DecOff off;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    off.k[i] = ((16 * i + r16) * D128 + 8 * g) * 2;
    off.v[i] = ((16 * i + 4 * g) * D128 + 8 * r16) * 2;
  }

  u32x4 qf[4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(R.q) + int64_t(j * G + (head_ok ? r16 : 0)) * D128;
#pragma unroll
    for (int c = 0; c < 4; c++) qf[c] = head_ok ? *reinterpret_cast<const u32x4*>(qp + 32 * c + 8 * g) : u32x4{0, 0, 0, 0};
  }
  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; dt++) oacc[dt] = f32x4{0, 0, 0, 0};
  float m_run = NEG_INF, l_run = 0.f;
  const float sl2 = args.scale_log2;

  DecK kr;
  DecV vr;
  int t0 = key_lo + ATT_KT * wave;
  if (t0 < key_hi) dec_load(kr, vr, R.a, R.b, a_al, j, t0, off);
  for (; t0 < key_hi; t0 += DEC_WAVES * ATT_KT) {
    // The LDS addresses below are loop invariant; hoisted out of the loop they would not fit
    // in registers next to two tiles, and their spill reloads would serialise every tile.
    // Offsetting the tile base by an opaque zero makes the compiler recompute them (a few
    // VALU operations per tile).
    int zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
    uint16_t* const Vw = Vt + zero;
    // ---- S^T = K Q^T (16 keys x 16 heads per group)
    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
      sacc[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < 4; c++) sacc[kt] = mfma_bf16(kr.k[kt][c], qf[c], sacc[kt]);
    }
    // ---- V -> fp16, transposed into this wave's LDS tile
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int grp = 4 * (q >> 1) + g, half = q & 1;
#pragma unroll
      for (int c = 0; c < 8; c++) {
        const int d = 8 * r16 + c;
        float x[4];
#pragma unroll
        for (int jj = 0; jj < 4; jj++) x[jj] = (c & 1) ? hi_bf(vr.v[q][jj][c >> 1]) : lo_bf(vr.v[q][jj][c >> 1]);
        u32x2 w;
        w.x = pack_h2(x[0], x[1]);
        w.y = pack_h2(x[2], x[3]);
        *reinterpret_cast<u32x2*>(Vw + d * ATT_KT + 8 * (grp ^ dec_sw(d)) + 4 * half) = w;
      }
    }
    // ---- next tile in flight while this one finishes (the scheduling barrier keeps the
    // loads from being hoisted above the last uses of the registers they overwrite)
    __builtin_amdgcn_sched_barrier(0);
    const int tn = t0 + DEC_WAVES * ATT_KT;
    if (tn < key_hi) dec_load(kr, vr, R.a, R.b, a_al, j, tn, off);

    // ---- scale, mask, online softmax per head (column l % 16)
    float mx = NEG_INF;
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int t = t0 + 16 * kt + 4 * g + jj;
        const bool vis = (t < key_hi) & ((t < a_n) | (t >= a_al));
        const float v = vis ? sacc[kt][jj] * sl2 : NEG_INF;
        sacc[kt][jj] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    // finite: key t0 of a processed tile is always visible (t0 < a_n or a_al <= t0 < key_hi)
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const float p = __builtin_amdgcn_exp2f(sacc[kt][jj] - m_new);
        sacc[kt][jj] = p;
        rs += p;
      }
    }
    rs += shfl_xor(rs, 16);
    rs += shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__any(alpha != 1.f)) {  // the running max rarely moves after the first tiles; x * 1 == x
#pragma unroll
      for (int dt = 0; dt < 8; dt++) oacc[dt] *= alpha;
    }

    // LDS operations of one wave complete in issue order; the fence keeps the compiler
    // from moving the fragment reads above the tile stores (and later stores above them).
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // ---- O^T += V^T P^T over 2 chunks of 32 keys, P as an fp16 hi/lo pair
#pragma unroll
    for (int kc = 0; kc < 2; kc++) {
      uint32_t h[4], lw[4];
      split_h2(sacc[2 * kc][0] * P_SCALE, sacc[2 * kc][1] * P_SCALE, h[0], lw[0]);
      split_h2(sacc[2 * kc][2] * P_SCALE, sacc[2 * kc][3] * P_SCALE, h[1], lw[1]);
      split_h2(sacc[2 * kc + 1][0] * P_SCALE, sacc[2 * kc + 1][1] * P_SCALE, h[2], lw[2]);
      split_h2(sacc[2 * kc + 1][2] * P_SCALE, sacc[2 * kc + 1][3] * P_SCALE, h[3], lw[3]);
      const u32x4 pb = u32x4{h[0], h[1], h[2], h[3]};
      const u32x4 pl = u32x4{lw[0], lw[1], lw[2], lw[3]};
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
        const int d = 16 * dt + r16;
        const u32x4 va = *reinterpret_cast<const u32x4*>(Vw + d * ATT_KT + 8 * ((4 * kc + g) ^ dec_sw(d)));
        oacc[dt] = mfma_f16(va, pb, oacc[dt]);
        oacc[dt] = mfma_f16(va, pl, oacc[dt]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }

  // ---- merge the four wave states in wave order; lane holds o[16dt + 4g + jj] of head l % 16
  float* red = reinterpret_cast<float*>(Vt);  // [G][DEC_RED]: m, l, o[D]
  if (head_ok) {
    float* rh = red + r16 * DEC_RED;
    if (g == 0) {
      rh[0] = m_run;
      rh[1] = l_run;
    }
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) rh[2 + 16 * dt + 4 * g + jj] = oacc[dt][jj] * P_UNSCALE;
    }
  }
  __syncthreads();
  const float* red0 = reinterpret_cast<const float*>(lds);
  for (int idx = tid; idx < G * (D128 + 2); idx += 256) {
    const int n = idx / (D128 + 2), e = idx - n * (D128 + 2);
    float mw[DEC_WAVES];
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; w++) {
      mw[w] = red0[w * (DEC_TILE / 2) + n * DEC_RED];
      M = fmaxf(M, mw[w]);
    }
    float acc = 0.f;
    if (e == 0) {
      acc = M;
    } else {
#pragma unroll
      for (int w = 0; w < DEC_WAVES; w++) {
        const float wt = mw[w] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
        acc = fmaf(red0[w * (DEC_TILE / 2) + n * DEC_RED + e], wt, acc);
      }
    }
    R.part[(int64_t(j * G + n) * R.s_total + (R.s_off + s)) * (D128 + 2) + e] = acc;
  }
}

// ---------------------------------------------------------------- fp32 (head_dim 64), VALU
// One workgroup (64 threads) per (request, KV head, query row, split).  Lane t
// scores key t0 + t of each 64-key tile; lane d accumulates o[d].  The key
// order and tile boundaries are fixed by absolute key index, so each row's
// result does not depend on the other rows of the call.
constexpr int D64 = 64;

__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnArgs args) {
  __shared__ float Kt[ATT_KT][D64 + 1];
  __shared__ float Vs[ATT_KT][D64];
  __shared__ float qs[D64];
  __shared__ float ps[ATT_KT];
  const int lane = threadIdx.x;
  const int z = blockIdx.z;
  if (z >= args.n_req) return;
  const AttnReq& R = args.r[z];
  const int Hkv = args.Hkv, G = args.G, Hq = args.Hq;
  const int j = blockIdx.x % Hkv, qr = blockIdx.x / Hkv;
  const int s = blockIdx.y;
  const int n_qrows = R.n_rows * G;
  if (qr >= n_qrows || s >= R.n_splits) return;
  const int qi = qr / G, hq = j * G + qr % G;
  const int n_keys = R.a.n + R.b.n + R.c.n;
  const int key_lo = s * args.split_len;
  const int lim = R.lim0 + qi;
  const int key_hi = min(min(key_lo + args.split_len, n_keys), lim + 1);
  const float* qp = static_cast<const float*>(R.q) + (int64_t(qi) * Hq + hq) * D64;
  qs[lane] = qp[lane];
  float m_run = NEG_INF, l_run = 0.f, o = 0.f;
  const float sl2 = args.scale_log2;
  for (int t0 = key_lo; t0 < key_hi; t0 += ATT_KT) {
    __syncthreads();
    for (int r = 0; r < ATT_KT; r++) {
      const int t = t0 + r;
      float kv = 0.f, vv = 0.f;
      if (t < n_keys) {
        kv = key_row<float, D64>(R, j, t, false)[lane];
        vv = key_row<float, D64>(R, j, t, true)[lane];
      }
      Kt[r][lane] = kv;
      Vs[r][lane] = vv;
    }
    __syncthreads();
    const int t = t0 + lane;
    float sc = 0.f;
    for (int d = 0; d < D64; d++) sc = fmaf(qs[d], Kt[lane][d], sc);
    const bool vis = t < n_keys && t <= lim;
    const float v = vis ? sc * sl2 : NEG_INF;
    float mx = v;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
    const float m_new = fmaxf(m_run, mx);
    const bool none = (m_new == NEG_INF);
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float p = none ? 0.f : __builtin_amdgcn_exp2f(v - m_new);
    float rs = p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) rs += shfl_xor(rs, off);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    ps[lane] = p;
    __syncthreads();
    float acc = 0.f;
    for (int r = 0; r < ATT_KT; r++) acc = fmaf(ps[r], Vs[r][lane], acc);
    o = o * alpha + acc;
  }
  float* dst = R.part + ((int64_t(qi) * Hq + hq) * R.s_total + (R.s_off + s)) * (D64 + 2);
  if (lane == 0) {
    dst[0] = m_run;
    dst[1] = l_run;
  }
  dst[2 + lane] = o;
}

// ---------------------------------------------------------------- combine
// One workgroup per (request, row, query head); thread d merges o[d] over the splits in
// ascending order.  The per-split loads are independent, so they are issued in unrolled
// chunks of CMB_CHUNK and only the accumulation runs in sequence.
constexpr int CMB_CHUNK = 16;

__global__ __launch_bounds__(128) void combine_kernel(const CombineArgs a) {
  const int z = blockIdx.y;
  if (z >= a.n_req) return;
  const int rh = blockIdx.x;  // row * Hq + hq
  const int D = a.head_dim;
  const int d = threadIdx.x;
  if (d >= D) return;
  const int64_t ps = D + 2;
  const float* p = a.part[z] + int64_t(rh) * a.s_total * ps;
  const int S = a.s_used[z];
  float M = NEG_INF;
  for (int s0 = 0; s0 < S; s0 += CMB_CHUNK) {
    float m[CMB_CHUNK];
#pragma unroll
    for (int i = 0; i < CMB_CHUNK; i++) m[i] = s0 + i < S ? p[(s0 + i) * ps] : NEG_INF;
#pragma unroll
    for (int i = 0; i < CMB_CHUNK; i++) M = fmaxf(M, m[i]);
  }
  float L = 0.f, O = 0.f;
  for (int s0 = 0; s0 < S; s0 += CMB_CHUNK) {
    float m[CMB_CHUNK], l[CMB_CHUNK], o[CMB_CHUNK];
#pragma unroll
    for (int i = 0; i < CMB_CHUNK; i++) {
      const bool ok = s0 + i < S;
      m[i] = ok ? p[(s0 + i) * ps] : NEG_INF;
      l[i] = ok ? p[(s0 + i) * ps + 1] : 0.f;
      o[i] = ok ? p[(s0 + i) * ps + 2 + d] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < CMB_CHUNK; i++) {
      if (s0 + i < S) {
        const float w = (m[i] == NEG_INF) ? 0.f : __builtin_amdgcn_exp2f(m[i] - M);
        L = fmaf(l[i], w, L);
        O = fmaf(o[i], w, O);
      }
    }
  }
  const float r = O / L;
  if (a.out_dtype == VC_BF16) {
    static_cast<uint16_t*>(a.out[z])[int64_t(rh) * D + d] = f2bf(r);
  } else {
    static_cast<float*>(a.out[z])[int64_t(rh) * D + d] = r;
  }
}

}  // namespace

vc_status launch_attn_decode(const AttnArgs& a, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (a.n_req <= 0 || a.max_splits <= 0) {
    VC_EVENTS_IF_EMPTY(ev_start, ev_stop, s);
    return VC_OK;
  }
  VC_REQUIRE(a.head_dim == 128 && a.G >= 1 && a.G <= 16 && a.split_len % (DEC_WAVES * ATT_KT) == 0, VC_ERR_UNSUPPORTED,
             "decode attention needs head_dim 128, at most 16 query heads per KV head, split a multiple of 256");
  for (int r = 0; r < a.n_req; r++) {
    const AttnReq& q = a.r[r];
    VC_REQUIRE(q.n_rows == 1, VC_ERR_UNSUPPORTED, "decode attention takes one query row per request");
    VC_REQUIRE(int64_t(q.a.n) * D128 * 2 < (int64_t(1) << 31) && int64_t(q.b.n) * D128 * 2 < (int64_t(1) << 31),
               VC_ERR_UNSUPPORTED, "decode attention: segment above 2 GiB per head");
    VC_REQUIRE(int64_t(q.n_splits) * a.split_len >= decode_keys(q.a.n, q.b.n), VC_ERR_ARG,
               "decode attention: %d splits do not cover the keys", q.n_splits);
  }
  hipExtLaunchKernelGGL(attn_decode_bf16_kernel, dim3(a.Hkv, a.max_splits, a.n_req), dim3(256), 0, s, ev_start,
                        ev_stop, 0, a);
  VC_LAUNCH_CHECK();
  return VC_OK;
}

vc_status launch_attn(const AttnArgs& a, int dtype, hipStream_t s, bool draft) {
  if (a.n_req <= 0 || a.max_splits <= 0) return VC_OK;
  if (dtype == VC_BF16) {
    VC_REQUIRE(a.head_dim == 128, VC_ERR_UNSUPPORTED, "bf16 attention needs head_dim 128 (got %d)", a.head_dim);
    (void)draft;
    int max_qrows = 0;
    for (int i = 0; i < a.n_req; i++) max_qrows = max(max_qrows, a.r[i].n_rows * a.G);
    // row blocks per wave: enough for the largest request up to 3 (a 192-row group)
    const int rpw = max(1, min(3, int(cdiv(max_qrows, ATT_RB))));
    const int n_groups = int(cdiv(max_qrows, ATT_RB * rpw));
    dim3 grid(a.Hkv * n_groups, a.max_splits, a.n_req);
    if (rpw == 1) hipLaunchKernelGGL(attn_rows_bf16_kernel<1>, grid, dim3(256), 0, s, a);
    else if (rpw == 2) hipLaunchKernelGGL(attn_rows_bf16_kernel<2>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(attn_rows_bf16_kernel<3>, grid, dim3(256), 0, s, a);
  } else {
    VC_REQUIRE(a.head_dim == 64, VC_ERR_UNSUPPORTED, "fp32 attention needs head_dim 64 (got %d)", a.head_dim);
    int max_qrows = 0;
    for (int i = 0; i < a.n_req; i++) max_qrows = max(max_qrows, a.r[i].n_rows * a.G);
    dim3 grid(a.Hkv * max_qrows, a.max_splits, a.n_req);
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(64), 0, s, a);
  }
  VC_LAUNCH_CHECK();
  return VC_OK;
}

vc_status launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.n_req <= 0) return VC_OK;
  dim3 grid(a.n_rows * a.Hq, a.n_req);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(128), 0, s, a);
  VC_LAUNCH_CHECK();
  return VC_OK;
}

}  // namespace vc
