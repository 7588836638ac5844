// Rows attention (verification, prefill, observation scores): split-K partials of many
// query rows over bf16 / fp32 key segments; the partials are merged by combine_kernel
// (attention.hip).
//
// bf16 kernel (head_dim 128), one workgroup = 4 waves = (request, KV head,
// group of up to 64 * RPW query rows, split).  Per 64-key tile the whole workgroup
// stages K (row major) and V (transposed, keys contiguous per channel) in LDS; each
// wave then computes, for each 16-row block it owns,
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
#include <type_traits>

#include "attention.h"
#include "bounds.h"

namespace vc {

namespace {

constexpr int D128 = 128;
// LDS tiles, 16-byte chunks XOR-swizzled within each row.  A ds_read_b128 is served in four
// passes of 16 lanes: per half-wave, the quads (4 lanes) whose index has even bit parity
// (lanes 0-3, 12-15, 20-23, 24-27) and those with odd parity (measured with the bank-conflict
// counter).  A fragment read takes row r = lane % 16 and chunk q + lane / 16, so a pass holds
// rows {0-3, 12-15} at one chunk and rows {4-11} at the next (or the reverse):
//   K (and the shared blocks' queries): 256-byte rows, chunk q stored at q ^ (r % 16), so each
//     pass covers the 16 chunk positions of the 256 bytes (all 64 banks) once;
//   V^T: 128-byte rows (two per 256 bytes), chunk q at q ^ ((r / 2) % 8), so each pass's rows of
//     either parity take eight different chunk positions.
constexpr int KS_PITCH = D128;   // bf16 per K row
constexpr int VT_PITCH = ATT_KT; // fp16 per V^T row
__device__ __forceinline__ int ks_off(int row, int chunk) { return row * KS_PITCH + 8 * (chunk ^ (row & 15)); }
__device__ __forceinline__ int vt_off(int row, int chunk) { return row * VT_PITCH + 8 * (chunk ^ ((row >> 1) & 7)); }
constexpr float P_SCALE = 1024.f;      // P is rounded to fp16 as P * 2^10
constexpr float P_LOG2 = 10.f;         // log2 of P_SCALE
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

// Where the 64 keys of tile t0 live when segment a is a token-drop mix of kept rows (on the
// GPU) and staged host rows: bit o of m set means key t0 + o is kept row c + (set bits of m
// below o); otherwise it is staged row t0 - c + (clear bits below o).  valid = the tile lies
// wholly in a mixed segment a.  Both words are uniform per (KV head, tile), so the kernel
// fetches them a tile ahead of the rows they locate.
struct TileMix {
  uint64_t m;
  int c;
  bool valid;
};

__device__ __forceinline__ TileMix tile_mix(const AttnReq& R, int j, int t0) {
  TileMix x{0, 0, false};
  if (R.mix.mask != nullptr && t0 + ATT_KT <= R.a.n) {
    const int64_t i = int64_t(j) * R.mix.nt + (t0 >> 6);
    const uint64_t m = R.mix.mask[i];
    // readfirstlane yields int: widen through uint32_t (no sign extension into the high word)
    const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(m >> 32)));
    const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(m)));
    x.m = (uint64_t(hi) << 32) | lo;
    x.c = __builtin_amdgcn_readfirstlane(R.mix.cnt[i]);
    x.valid = true;
  }
  return x;
}

// K: thread (kr = tid/16, ch = tid%16) loads 16-byte chunk ch of keys kr + 16e (e = 0..3):
//    sixteen consecutive lanes move one whole 256-byte row (coalesced in HBM, and their LDS
//    stores cover all banks once).
// V: thread (dc = tid/16, kg = tid%16) loads channels 8dc..8dc+7 of keys 4kg..4kg+3.
// mix: tile_mix(R, j, t0).
__device__ __forceinline__ void load_tile_bf16(TileRegs& r, const AttnReq& R, int j, int t0, int n_keys, int tid,
                                               const TileMix& mix) {
  const int kr = tid >> 4, ch = tid & 15, dc = tid >> 4, kg = tid & 15;
  const uint16_t* kb;
  const uint16_t* vb;
  if (tile_plain(R, j, t0, n_keys, kb, vb)) {  // uniform across the workgroup
#pragma unroll
    for (int e = 0; e < 4; e++) r.k[e] = ld_nt(kb + (kr + 16 * e) * D128 + 8 * ch);
#pragma unroll
    for (int e = 0; e < 4; e++) r.v[e] = ld_nt(vb + (4 * kg + e) * D128 + 8 * dc);
    return;
  }
  if (mix.valid) {  // uniform: every row in the kept / staged mix of segment a
    // lane o of each wave locates key t0 + o (one popcount); each thread then takes the rows of
    // its eight loads from the lanes that located them (the top bit marks a kept row)
    // (set bits of m below this lane: v_mbcnt, so no per-lane 64-bit mask is kept in registers)
    const int o = tid & 63;
    const uint32_t m_lo = uint32_t(mix.m), m_hi = uint32_t(mix.m >> 32);
    const int below = int(__builtin_amdgcn_mbcnt_hi(m_hi, __builtin_amdgcn_mbcnt_lo(m_lo, 0u)));
    const bool kept = ((o < 32 ? m_lo >> o : m_hi >> (o - 32)) & 1u) != 0;
    const uint32_t handle = kept ? (uint32_t(mix.c + below) | 0x80000000u) : uint32_t(t0 - mix.c + o - below);
    const uint16_t* kk = static_cast<const uint16_t*>(R.mix.k) + j * R.mix.hstride;
    const uint16_t* sk = static_cast<const uint16_t*>(R.a.k) + j * R.a.hstride;
    const uint16_t* kv = static_cast<const uint16_t*>(R.mix.v) + j * R.mix.hstride;
    const uint16_t* sv = static_cast<const uint16_t*>(R.a.v) + j * R.a.hstride;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const uint32_t h = uint32_t(__shfl(int(handle), kr + 16 * e, 64));
      const uint16_t* base = (h & 0x80000000u) ? kk : sk;
      r.k[e] = ld_nt(base + int64_t(h & 0x7fffffffu) * D128 + 8 * ch);
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const uint32_t h = uint32_t(__shfl(int(handle), 4 * kg + e, 64));
      const uint16_t* base = (h & 0x80000000u) ? kv : sv;
      r.v[e] = ld_nt(base + int64_t(h & 0x7fffffffu) * D128 + 8 * dc);
    }
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
  for (int e = 0; e < 4; e++) *reinterpret_cast<u32x4*>(Ks + ks_off(kr + 16 * e, ch)) = r.k[e];
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
    *reinterpret_cast<u32x2*>(Vt + vt_off(8 * dc + c, slot >> 3) + (slot & 7)) = out;
  }
}

// Rows kernel (verification, prefill, observation scores): workgroup = 4 waves =
// (request, KV head, group of query rows, split).  A group holds up to 4 RPW "own" row blocks
// of 16 rows -- wave w keeps the state of blocks w and w + 4 in registers -- followed by up to
// JMAX "shared" blocks that the four waves compute together: for the block's scores wave w takes
// keys 16w .. 16w + 15 of each tile, the waves exchange the scores through LDS, each then runs
// the block's online softmax on the whole tile (all four identically) and accumulates the
// output channels 32w .. 32w + 31.  A 33-row verification of 4 GQA heads (132 rows) is eight
// own blocks and one shared block, so the four waves issue the same MFMA work; every K/V tile
// staged in LDS serves all the rows of the group.  A row's arithmetic is the same whichever
// kind of block or group holds it: the same MFMAs in the same order for its scores and for
// each output channel, the same softmax sequence.
template <int RPW, int JMAX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_rows_bf16_kernel(
    const AttnArgs args) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[ATT_KT * KS_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D128 * VT_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Qj[JMAX > 0 ? JMAX * ATT_MB * KS_PITCH : 1];  // shared blocks' queries
  __shared__ __attribute__((aligned(16))) f32x4 Sx[JMAX > 0 ? JMAX * 4 * 64 : 1];  // [block][16-key slice][lane]
  constexpr int OWN_ROWS = ATT_RB * RPW;
  constexpr int GROUP_ROWS = OWN_ROWS + ATT_MB * JMAX;
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
  // shared blocks in use (uniform): those holding at least one row
  const int nj = JMAX > 0 ? min(JMAX, max(0, (n_qrows - (qr0 + OWN_ROWS) + ATT_MB - 1) / ATT_MB)) : 0;

  auto q_row = [&](int qr) -> const uint16_t* {  // query row qr (row qr / G, head j G + qr % G)
    const int qi = qr / G, hq = j * G + qr % G;
    return static_cast<const uint16_t*>(R.q) + (int64_t(qi) * Hq + hq) * D128;
  };

  // per own row block b of this wave: the lane's query row qr0 + 16 (wave + 4b) + lane % 16, its
  // query fragments and softmax state; the row indices are recomputed where needed
  const int qr_lane = qr0 + ATT_MB * wave + (lane & 15);
  auto blk_on = [&](int b) { return qr0 + ATT_MB * (wave + 4 * b) < n_qrows; };  // uniform per wave
  int n_act = 0;  // active own blocks 0 .. n_act - 1 of this wave
#pragma unroll
  for (int b = 0; b < RPW; b++) n_act += blk_on(b) ? 1 : 0;
  u32x4 qf[RPW][4];
  f32x4 oacc[RPW][8];
  float m_run[RPW], l_run[RPW];
#pragma unroll
  for (int b = 0; b < RPW; b++) {
    const int qr = qr_lane + ATT_RB * b;
    const bool row_ok = qr < n_qrows;
    const uint16_t* qp = q_row(row_ok ? qr : 0);
#pragma unroll
    for (int c = 0; c < 4; c++)
      qf[b][c] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 32 * c + 8 * grp) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int dt = 0; dt < 8; dt++) oacc[b][dt] = f32x4{0, 0, 0, 0};
    m_run[b] = NEG_INF;
    l_run[b] = 0.f;
  }
  // shared blocks: queries into LDS (thread = one 16-byte chunk of one row), and per block this
  // wave's two output channel tiles and the block's softmax state (the same in every wave)
  f32x4 oj[JMAX > 0 ? JMAX : 1][2];
  float mj[JMAX > 0 ? JMAX : 1], lj[JMAX > 0 ? JMAX : 1];
#pragma unroll
  for (int jb = 0; jb < JMAX; jb++) {
    if (jb < nj) {
      const int r = tid >> 4, ch = tid & 15;
      const int qr = qr0 + OWN_ROWS + ATT_MB * jb + r;
      *reinterpret_cast<u32x4*>(Qj + ks_off(jb * ATT_MB + r, ch)) =
          qr < n_qrows ? *reinterpret_cast<const u32x4*>(q_row(qr) + 8 * ch) : u32x4{0, 0, 0, 0};
    }
    oj[jb][0] = oj[jb][1] = f32x4{0, 0, 0, 0};
    mj[jb] = NEG_INF;
    lj[jb] = 0.f;
  }
  const float sl2 = args.scale_log2;

  // a tile at or below lim_all is visible to every row of the group (and holds no key past
  // the last); padding rows (past n_qrows) compute on zero queries and are never written
  const int lim_all = min(R.lim0 + qr0 / G, n_keys - 1);

  // Online softmax of one block's 64-key tile held in the MFMA output layout (row qr = the lane's
  // row, keys 16kt + 4 grp + jj): masks, the running max and sum, and P' = 2^10 p in place.
  // Scores stay unscaled until the exponent: p' = 2^(s * scale_log2 - m + 10) in one fma per key,
  // m and the running sum in the scaled domain (the 2^10 is removed when the partial is written).
  // Returns the factor the block's accumulators take.
  auto softmax = [&](f32x4 (&sa)[4], float& m_run_, float& l_run_, int qr, int t0, bool full) -> float {
    float mx = NEG_INF;
    if (full) {
#pragma unroll
      for (int kt = 0; kt < 4; kt++) mx = fmaxf(mx, fmaxf(fmaxf(sa[kt][0], sa[kt][1]), fmaxf(sa[kt][2], sa[kt][3])));
    } else {
      const int lim = qr < n_qrows ? min(R.lim0 + qr / G, n_keys - 1) : -1;
#pragma unroll
      for (int kt = 0; kt < 4; kt++) {
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int t = t0 + 16 * kt + 4 * grp + jj;
          const bool vis = t <= lim;
          sa[kt][jj] = vis ? sa[kt][jj] : NEG_INF;
          mx = fmaxf(mx, sa[kt][jj]);
        }
      }
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run_, mx * sl2);
    // no visible key yet (masked tiles only): nothing to add, state unchanged
    const bool none = !full && m_new == NEG_INF;
    const float nb = none ? 0.f : P_LOG2 - m_new;
    const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run_ - m_new);
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sa[kt][jj], sl2, nb));
        sa[kt][jj] = p;
        rs += p;
      }
    }
    rs += shfl_xor(rs, 16);
    rs += shfl_xor(rs, 32);
    l_run_ = l_run_ * alpha + rs;
    m_run_ = m_new;
    return alpha;
  };
  // P' of 32 keys (chunk kc of the tile) as fp16 hi / lo MFMA B fragments
  auto p_frags = [&](const f32x4 (&sa)[4], int kc, u32x4& pb, u32x4& pl) {
    uint32_t h[4], lw[4];
    split_h2(sa[2 * kc][0], sa[2 * kc][1], h[0], lw[0]);
    split_h2(sa[2 * kc][2], sa[2 * kc][3], h[1], lw[1]);
    split_h2(sa[2 * kc + 1][0], sa[2 * kc + 1][1], h[2], lw[2]);
    split_h2(sa[2 * kc + 1][2], sa[2 * kc + 1][3], h[3], lw[3]);
    pb = u32x4{h[0], h[1], h[2], h[3]};
    pl = u32x4{lw[0], lw[1], lw[2], lw[3]};
  };

  TileRegs regs;
  TileMix mix_next = tile_mix(R, j, key_lo + ATT_KT);
  if (key_lo < key_hi) load_tile_bf16(regs, R, j, key_lo, n_keys, tid, tile_mix(R, j, key_lo));
  for (int t0 = key_lo; t0 < key_hi; t0 += ATT_KT) {
    __syncthreads();
    store_tile_bf16(regs, Ks, Vt, tid);
    __syncthreads();
    if (t0 + ATT_KT < key_hi) {
      load_tile_bf16(regs, R, j, t0 + ATT_KT, n_keys, tid, mix_next);
      mix_next = tile_mix(R, j, t0 + 2 * ATT_KT);
    }
    const bool full = t0 + ATT_KT - 1 <= lim_all;  // uniform

    // Own row blocks [B0, B0 + NB) of this wave (NB <= 2): each K and V^T fragment read from LDS
    // feeds the MFMAs of all NB blocks.  Per block, the MFMA sequence and the softmax arithmetic
    // are the same whichever blocks share the pass.
    auto blocks = [&](auto b0v, auto nbv) {
      constexpr int B0 = decltype(b0v)::value, NB = decltype(nbv)::value;
      // ---- S^T = K Q^T over 4 sub-tiles of 16 keys
      f32x4 sacc[NB][4];
#pragma unroll
      for (int b = 0; b < NB; b++)
#pragma unroll
        for (int kt = 0; kt < 4; kt++) sacc[b][kt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int kt = 0; kt < 4; kt++) {
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(Ks + ks_off(16 * kt + (lane & 15), 4 * c + grp));
#pragma unroll
          for (int b = 0; b < NB; b++) sacc[b][kt] = mfma_bf16(ka, qf[B0 + b][c], sacc[b][kt]);
        }
      }
      // the softmax phase at a raised wave priority, the MFMA phases at the normal one, so the two
      // waves of a SIMD tend to alternate between them instead of meeting in the same phase
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int b = 0; b < NB; b++) {
        const float alpha = softmax(sacc[b], m_run[B0 + b], l_run[B0 + b], qr_lane + ATT_RB * (B0 + b), t0, full);
        if (__any(alpha != 1.f)) {  // x * 1 == x: skip the rescale when no running max moved
#pragma unroll
          for (int dt = 0; dt < 8; dt++) oacc[B0 + b][dt] *= alpha;
        }
      }
      // ---- O^T += V^T P^T over 2 chunks of 32 keys, P as an fp16 hi/lo pair
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int kc = 0; kc < 2; kc++) {
        u32x4 pb[NB], pl[NB];
#pragma unroll
        for (int b = 0; b < NB; b++) p_frags(sacc[b], kc, pb[b], pl[b]);
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
          const u32x4 va = *reinterpret_cast<const u32x4*>(Vt + vt_off(16 * dt + (lane & 15), 4 * kc + grp));
#pragma unroll
          for (int b = 0; b < NB; b++) {
            oacc[B0 + b][dt] = mfma_f16(va, pb[b], oacc[B0 + b][dt]);
            oacc[B0 + b][dt] = mfma_f16(va, pl[b], oacc[B0 + b][dt]);
          }
        }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if constexpr (RPW >= 2) {
      if (n_act >= 2) blocks(I0{}, I2{});
      else if (n_act == 1) blocks(I0{}, I1{});
    } else {
      if (n_act == 1) blocks(I0{}, I1{});
    }

    // ---- shared blocks, scores (after the own blocks, whose registers are then free): this
    // wave's 16 keys (sub-tile kt = wave), the same MFMAs an own block runs for that sub-tile,
    // out to LDS
#pragma unroll
    for (int jb = 0; jb < JMAX; jb++) {
      if (jb < nj) {
        f32x4 sj = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(Ks + ks_off(16 * wave + (lane & 15), 4 * c + grp));
          const u32x4 qb = *reinterpret_cast<const u32x4*>(Qj + ks_off(jb * ATT_MB + (lane & 15), 4 * c + grp));
          sj = mfma_bf16(ka, qb, sj);
        }
        Sx[(jb * 4 + wave) * 64 + lane] = sj;
      }
    }

    // ---- shared blocks: the whole tile's scores from the four waves, softmax, this wave's
    // output channel tiles 2 wave and 2 wave + 1
    if (nj > 0) {  // uniform
      __syncthreads();
#pragma unroll
      for (int jb = 0; jb < JMAX; jb++) {
        if (jb < nj) {
          f32x4 sa[4];
#pragma unroll
          for (int kt = 0; kt < 4; kt++) sa[kt] = Sx[(jb * 4 + kt) * 64 + lane];
          const float alpha = softmax(sa, mj[jb], lj[jb], qr0 + OWN_ROWS + ATT_MB * jb + (lane & 15), t0, full);
          if (__any(alpha != 1.f)) {
            oj[jb][0] *= alpha;
            oj[jb][1] *= alpha;
          }
#pragma unroll
          for (int kc = 0; kc < 2; kc++) {
            u32x4 pb, pl;
            p_frags(sa, kc, pb, pl);
#pragma unroll
            for (int dd = 0; dd < 2; dd++) {
              const int dt = 2 * wave + dd;
              const u32x4 va = *reinterpret_cast<const u32x4*>(Vt + vt_off(16 * dt + (lane & 15), 4 * kc + grp));
              oj[jb][dd] = mfma_f16(va, pb, oj[jb][dd]);
              oj[jb][dd] = mfma_f16(va, pl, oj[jb][dd]);
            }
          }
        }
      }
    }
  }

  // ---- partials (m, l, o): own blocks, lane holds o[16dt + 4g + jj]
  auto part_of = [&](int qr) -> float* {
    const int qi = qr / G, hq = j * G + qr % G;
    return R.part + ((int64_t(qi) * Hq + hq) * R.s_total + (R.s_off + s)) * (D128 + 2);
  };
#pragma unroll
  for (int b = 0; b < RPW; b++) {
    const int qr = qr_lane + ATT_RB * b;
    if (!blk_on(b) || qr >= n_qrows) continue;
    float* dst = part_of(qr);
    if (grp == 0) {
      dst[0] = m_run[b];
      dst[1] = l_run[b] * P_UNSCALE;
    }
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) dst[2 + 16 * dt + 4 * grp + jj] = oacc[b][dt][jj] * P_UNSCALE;
    }
  }
  // shared blocks: each wave its two channel tiles, wave 0 the row's (m, l)
#pragma unroll
  for (int jb = 0; jb < JMAX; jb++) {
    const int qr = qr0 + OWN_ROWS + ATT_MB * jb + (lane & 15);
    if (jb >= nj || qr >= n_qrows) continue;
    float* dst = part_of(qr);
    if (wave == 0 && grp == 0) {
      dst[0] = mj[jb];
      dst[1] = lj[jb] * P_UNSCALE;
    }
#pragma unroll
    for (int dd = 0; dd < 2; dd++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) dst[2 + 16 * (2 * wave + dd) + 4 * grp + jj] = oj[jb][dd][jj] * P_UNSCALE;
    }
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

}  // namespace

vc_status launch_attn(const AttnArgs& a, int dtype, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (a.n_req <= 0 || a.max_splits <= 0) {
    VC_EVENTS_IF_EMPTY(ev_start, ev_stop, s);
    return VC_OK;
  }
  int max_qrows = 0;
  for (int i = 0; i < a.n_req; i++) max_qrows = max(max_qrows, a.r[i].n_rows * a.G);
  if (dbg_on()) {
    const int eb = dtype == VC_BF16 ? 2 : 4;
    for (int i = 0; i < a.n_req; i++)
      if (vc_status st = dbg_attn_req("attn_rows", a.r[i], a.Hq, a.Hkv, a.head_dim, eb)) return st;
    if (dbg_dry()) return VC_OK;
  }
  if (dtype == VC_BF16) {
    VC_REQUIRE(a.head_dim == 128, VC_ERR_UNSUPPORTED, "bf16 attention needs head_dim 128 (got %d)", a.head_dim);
    // row groups: up to 64 rows (one own block per wave); up to 144 (two own blocks per wave and
    // one shared block: a verification of up to 36 rows of 4 GQA heads in one group); beyond,
    // 128-row groups (prefill)
    if (max_qrows <= ATT_RB) {
      dim3 grid(a.Hkv, a.max_splits, a.n_req);
      hipExtLaunchKernelGGL((attn_rows_bf16_kernel<1, 0>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, a);
    } else if (max_qrows <= 2 * ATT_RB + ATT_MB) {
      dim3 grid(a.Hkv, a.max_splits, a.n_req);
      hipExtLaunchKernelGGL((attn_rows_bf16_kernel<2, 1>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, a);
    } else {
      dim3 grid(a.Hkv * int(cdiv(max_qrows, 2 * ATT_RB)), a.max_splits, a.n_req);
      hipExtLaunchKernelGGL((attn_rows_bf16_kernel<2, 0>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, a);
    }
  } else {
    VC_REQUIRE(a.head_dim == 64, VC_ERR_UNSUPPORTED, "fp32 attention needs head_dim 64 (got %d)", a.head_dim);
    dim3 grid(a.Hkv * max_qrows, a.max_splits, a.n_req);
    hipExtLaunchKernelGGL(attn_f32_kernel, grid, dim3(64), 0, s, ev_start, ev_stop, 0, a);
  }
  VC_LAUNCH_CHECK();
  return VC_OK;
}

}  // namespace vc
