// Draft-step attention over bf16 key segments (one query row per request) and the
// fixed-order combine of split-K partials; the many-row kernels are in
// attention_rows.hip, the quantized-cache decode in attention_quant.hip.
// QK^T is bf16 x bf16 with exact products.  In P.V the draft kernel keeps V in bf16 (any
// finite bf16 value) and carries P as a bf16 hi/lo pair (two MFMAs): hi = P rounded to bf16,
// lo = the remainder rounded to bf16, so each weight keeps about 17 significant bits.
#include "attention.h"
#include "bounds.h"

namespace vc {

namespace {

constexpr int D128 = 128;

// ---------------------------------------------------------------- bf16 decode, one query row
// Draft steps attend with a single query row per request, so a 64-row block would leave
// three of four waves idle.  Here one workgroup = 4 waves = (request, KV head, split) and
// wave w streams the 64-key tiles w, w + 4, w + 8, ... of the split on its own, with its own
// online softmax; the four states are merged in wave order at the end (fixed order, so the
// result does not depend on timing).  The G query heads of the KV head are the 16 MFMA
// columns.  K goes from HBM straight into A fragments (lane l: key l%16 of a 16-key group,
// channels 8(l/16)..+8 of a 32-channel chunk); V passes through a 16 KB LDS tile per wave,
// stored as loaded and read back transposed (below).  A wave issues the next tile's loads as
// soon as the current tile's registers are consumed, so its softmax and P.V overlap the next
// fetch; KV loads are non-temporal (every byte is read once).
// V tile layout: the wave's 64 keys as rows of 256 bytes (bf16, as in the cache); the eight
// 32-byte chunks of row t (16 channels each) sit in the order chunk ^ (t & 7), so eight
// consecutive rows put one channel chunk on eight different bank groups.  Lane (r16, g)
// stores its 16-byte pieces (key 16q + 4g + jj, channels 8 r16 .. + 8) with one ds_write_b128
// each.  The V^T fragments come back with the gfx950 LDS transpose read (ds_read_b64_tr_b16):
// in each 16-lane group, lane i of the result holds element i & 3 of the 8-byte pieces that
// lanes i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12 addressed.  Lane s of group g therefore
// addresses channels 16 dt + 4 (s & 3) .. + 4 of key row 4g + s / 4 (plus the 16-key half h of
// 32-key chunk kc), and lane m of the group receives channel 16 dt + m of keys 4g + 0..3: the
// four keys its P^T fragment holds in that half.
constexpr int DEC_WAVES = 4;
constexpr int DEC_TILE = D128 * ATT_KT;  // bf16 per wave LDS tile
constexpr int DEC_RED = D128 + 4;        // floats per head in the merge buffer

struct DecK {
  u32x4 k[4][4];  // [16-key group kt][32-channel chunk c]
};
struct DecV {
  u32x4 v[4][4];  // [16-key group q][key 4g + jj within it: jj]
};

// byte offset of (key row t, channel c) in a wave's V tile
constexpr int dec_v_addr(int t, int c) { return 256 * t + 32 * ((c >> 4) ^ (t & 7)) + 2 * (c & 15); }

// The kernel forms the tile's store and transpose-read addresses as (lane base) ^ (compile-time
// XOR) + (compile-time offset).  This checks, for every lane and access, that the stores put
// each piece where the layout says, and that the transpose reads (with the result lane mapping
// above) deliver to lane (m, g) channel 16 dt + m of keys 32 kc + 16 h + 4 g + e, e = 0..3, all
// inside the wave's 16 KB tile.
constexpr bool dec_tr_addressing_ok() {
  for (int lane = 0; lane < 64; lane++) {
    const int r16 = lane & 15, g = lane >> 4;
    const int st_lane = 1024 * g + 32 * ((r16 >> 1) ^ (4 * (g & 1))) + 16 * (r16 & 1);
    for (int q = 0; q < 4; q++) {
      for (int jj = 0; jj < 4; jj++) {
        const int got = (st_lane ^ (32 * jj)) + 4096 * q + 256 * jj;
        if (got != dec_v_addr(16 * q + 4 * g + jj, 8 * r16) || got + 16 > 2 * DEC_TILE) return false;
      }
    }
    for (int kc = 0; kc < 2; kc++) {
      for (int h = 0; h < 2; h++) {
        for (int dt = 0; dt < 8; dt++) {
          for (int e = 0; e < 4; e++) {
            const int src = 16 * g + (r16 >> 2) + 4 * e;  // the lane whose piece element e comes from
            const int rd_src = 256 * (src >> 2) + 32 * ((src >> 2) & 7) + 8 * (src & 3);
            const int addr = (rd_src ^ (32 * dt)) + 8192 * kc + 4096 * h;
            if (addr + 8 > 2 * DEC_TILE) return false;
            if (addr + 2 * (r16 & 3) != dec_v_addr(32 * kc + 16 * h + 4 * g + e, 16 * dt + r16)) return false;
          }
        }
      }
    }
  }
  return true;
}
static_assert(dec_tr_addressing_ok(), "decode V tile addressing does not match the layout");

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

  // LDS byte offsets of this lane's V stores and transpose reads (see the tile layout above):
  // the chunk swizzle is an XOR, (lane part) ^ (compile-time part), and the row an access touches
  // is the lane part plus a compile-time multiple of the row pitch, so each access is one XOR of
  // a lane base and an immediate offset.  The wave's tile starts on a 16 KB boundary and the
  // XORed bits (5-6 for stores, 5-7 for reads) are the chunk field, so the XOR never carries.
  //   store (key 16 q + 4 g + jj, channels 8 r16 .. + 8): (st_lane ^ 32 jj) + 4096 q + 256 jj
  //   read (half h of 32-key chunk kc, channels of 16-block dt): (rd_lane ^ 32 dt) + 8192 kc + 4096 h
  uint8_t* const lds8 = reinterpret_cast<uint8_t*>(lds);
  const uint32_t tile_base = uint32_t(wave) * (DEC_TILE * 2);
  const uint32_t st_lane = tile_base + 1024 * g + 32 * ((r16 >> 1) ^ (4 * (g & 1))) + 16 * (r16 & 1);
  const uint32_t rd_lane = tile_base + 256 * (lane >> 2) + 32 * ((lane >> 2) & 7) + 8 * (lane & 3);
  // a tile is wholly visible when it ends at or before key_hi and lies in the visible part of
  // its segment (segment a's keys below a_n, or segment b)
  const int a_vis_end = min(a_n, key_hi);

  DecK kr;
  DecV vr;
  int t0 = key_lo + ATT_KT * wave;
  if (t0 < key_hi) dec_load(kr, vr, R.a, R.b, a_al, j, t0, off);
  for (; t0 < key_hi; t0 += DEC_WAVES * ATT_KT) {
    // The lane bases are loop invariant; the twelve XORed addresses hoisted out of the loop would
    // not fit in registers next to two tiles (their spill reloads would serialise every tile), so
    // an opaque copy per tile makes the compiler form them again (twelve VALU operations).
    uint32_t st = st_lane, rd = rd_lane;
    asm volatile("" : "+v"(st), "+v"(rd));
    // ---- S^T = K Q^T (16 keys x 16 heads per group)
    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
      sacc[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int c = 0; c < 4; c++) sacc[kt] = mfma_bf16(kr.k[kt][c], qf[c], sacc[kt]);
    }
    // ---- V rows into this wave's LDS tile as they are
#pragma unroll
    for (int q = 0; q < 4; q++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++)
        *reinterpret_cast<u32x4*>(lds8 + (st ^ (32u * jj)) + (4096 * q + 256 * jj)) = vr.v[q][jj];
    }
    // ---- next tile in flight while this one finishes (the scheduling barrier keeps the
    // loads from being hoisted above the last uses of the registers they overwrite)
    __builtin_amdgcn_sched_barrier(0);
    const int tn = t0 + DEC_WAVES * ATT_KT;
    if (tn < key_hi) dec_load(kr, vr, R.a, R.b, a_al, j, tn, off);

    // softmax at a raised wave priority, P.V at the normal one: the two waves of a SIMD tend to
    // alternate between the VALU and the MFMA phase
    __builtin_amdgcn_s_setprio(1);
    // ---- mask, online softmax per head (column l % 16).  Scores stay unscaled until the
    // exponent: p = 2^(s * scale_log2 - m), one fma per key; m is kept in scaled (log2) units
    const bool full = t0 + ATT_KT <= key_hi && (t0 + ATT_KT <= a_vis_end || t0 >= a_al);  // uniform
    if (!full) {
#pragma unroll
      for (int kt = 0; kt < 4; kt++) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int t = t0 + 16 * kt + 4 * g + jj;
          const bool vis = (t < key_hi) & ((t < a_n) | (t >= a_al));
          sacc[kt][jj] = vis ? sacc[kt][jj] : NEG_INF;
        }
      }
    }
    float mx = NEG_INF;
#pragma unroll
    for (int kt = 0; kt < 4; kt++)
      mx = fmaxf(mx, fmaxf(fmaxf(sacc[kt][0], sacc[kt][1]), fmaxf(sacc[kt][2], sacc[kt][3])));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    // finite: key t0 of a processed tile is always visible (t0 < a_n or a_al <= t0 < key_hi)
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float nb = -m_new;
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][jj], sl2, nb));
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
    __builtin_amdgcn_s_setprio(0);
    // ---- O^T += V^T P^T over 2 chunks of 32 keys, P as a bf16 hi/lo pair
#pragma unroll
    for (int kc = 0; kc < 2; kc++) {
      uint32_t h[4], lw[4];
      split_bf2(sacc[2 * kc][0], sacc[2 * kc][1], h[0], lw[0]);
      split_bf2(sacc[2 * kc][2], sacc[2 * kc][3], h[1], lw[1]);
      split_bf2(sacc[2 * kc + 1][0], sacc[2 * kc + 1][1], h[2], lw[2]);
      split_bf2(sacc[2 * kc + 1][2], sacc[2 * kc + 1][3], h[3], lw[3]);
      const u32x4 pb = u32x4{h[0], h[1], h[2], h[3]};
      const u32x4 pl = u32x4{lw[0], lw[1], lw[2], lw[3]};
#pragma unroll
      for (int dt = 0; dt < 8; dt++) {
        const uint32_t a0 = (rd ^ (32u * dt)) + 8192 * kc;
        const u32x2 v0 = lds_read_tr16(lds8 + a0), v1 = lds_read_tr16(lds8 + a0 + 4096);
        const u32x4 va = u32x4{v0.x, v0.y, v1.x, v1.y};
        oacc[dt] = mfma_bf16(va, pb, oacc[dt]);
        oacc[dt] = mfma_bf16(va, pl, oacc[dt]);
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
      for (int jj = 0; jj < 4; jj++) rh[2 + 16 * dt + 4 * g + jj] = oacc[dt][jj];
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

vc_status dbg_kv_seg(const char* kernel, const char* what, const KVSeg& g, int Hkv, int D, int eb, int64_t rows) {
  if (rows <= 0) return VC_OK;
  char wk[96], wv[96];
  snprintf(wk, sizeof(wk), "%s K rows", what);
  snprintf(wv, sizeof(wv), "%s V rows", what);
  return dbg_check(kernel, {dbg_2d(wk, g.k, g.hstride * eb, rows * D * eb, Hkv),
                            dbg_2d(wv, g.v, g.hstride * eb, rows * D * eb, Hkv)});
}

vc_status dbg_attn_req(const char* kernel, const AttnReq& R, int Hq, int Hkv, int D, int eb) {
  if (R.s_off < 0 || R.s_off + R.n_splits > R.s_total)
    return dbg_fail("%s: partial slots %d..%d beyond the %d per row", kernel, R.s_off, R.s_off + R.n_splits - 1,
                    R.s_total);
  vc_status st = dbg_check(kernel, {{"queries", R.q, int64_t(R.n_rows) * Hq * D * eb},
                                    {"partials", R.part, int64_t(R.n_rows) * Hq * R.s_total * (D + 2) * 4}});
  if (st) return st;
  if (R.mix.mask) {
    // token-drop split of segment a: kept rows [0, kk) on the device, the other a.n - kk staged
    const int64_t kk = R.mix.hstride / D;
    if (int64_t(R.mix.nt) * 64 < R.a.n) return dbg_fail("%s: tile map of %d tiles for %d positions", kernel, R.mix.nt, R.a.n);
    if (kk > R.a.n) return dbg_fail("%s: %lld kept rows for %d positions", kernel, (long long)kk, R.a.n);
    const KVSeg kept{R.mix.k, R.mix.v, R.mix.hstride, 0, 0};
    if ((st = dbg_kv_seg(kernel, "kept prompt", kept, Hkv, D, eb, kk))) return st;
    if ((st = dbg_kv_seg(kernel, "staged prompt", R.a, Hkv, D, eb, R.a.n - kk))) return st;
    if ((st = dbg_check(kernel, {{"kept-tile masks", R.mix.mask, int64_t(Hkv) * R.mix.nt * 8},
                                 {"kept-tile counts", R.mix.cnt, int64_t(Hkv) * R.mix.nt * 4}})))
      return st;
  } else if ((st = dbg_kv_seg(kernel, "segment a", R.a, Hkv, D, eb, R.a.n))) {
    return st;
  }
  if ((st = dbg_kv_seg(kernel, "segment b", R.b, Hkv, D, eb, R.b.n))) return st;
  return dbg_kv_seg(kernel, "segment c", R.c, Hkv, D, eb, R.c.n);
}

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
    if (dbg_on()) {
      AttnReq d = q;
      d.c.n = 0;  // the decode kernel reads segments a and b only
      d.mix.mask = nullptr;
      if (vc_status st = dbg_attn_req("attn_decode_bf16", d, a.Hq, a.Hkv, 128, 2)) return st;
    }
  }
  if (dbg_dry()) return VC_OK;
  hipExtLaunchKernelGGL(attn_decode_bf16_kernel, dim3(a.Hkv, a.max_splits, a.n_req), dim3(256), 0, s, ev_start,
                        ev_stop, 0, a);
  VC_LAUNCH_CHECK();
  return VC_OK;
}


vc_status launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.n_req <= 0) return VC_OK;
  if (dbg_on()) {
    const int64_t rows = int64_t(a.n_rows) * a.Hq, ob = a.out_dtype == VC_BF16 ? 2 : 4;
    for (int r = 0; r < a.n_req; r++) {
      if (a.s_used[r] > a.s_total) return dbg_fail("combine: %d slots used of %d", a.s_used[r], a.s_total);
      if (vc_status st = dbg_check("combine", {{"partials", a.part[r], rows * a.s_total * (a.head_dim + 2) * 4},
                                               {"output", a.out[r], rows * a.head_dim * ob}}))
        return st;
    }
    if (dbg_dry()) return VC_OK;
  }
  dim3 grid(a.n_rows * a.Hq, a.n_req);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(128), 0, s, a);
  VC_LAUNCH_CHECK();
  return VC_OK;
}

}  // namespace vc
