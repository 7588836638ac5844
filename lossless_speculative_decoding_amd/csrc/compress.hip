// Compressors ("The Uniform Compressor Interface", VeriCache Guide): per-group
// quantization with bit packing, and token dropping by observed attention or by key norm.
//
// Quantization arithmetic is IEEE float32 step by step (no contraction) so
// that codes, scales and zeros are bit-identical to the reference definition:
//   zero = fp16(min); scale = fp16((max - min) / (2^b - 1));
//   code = scale == 0 ? 0 : clamp(rint((x - zero) / scale), 0, 2^b - 1).
#include "attention.h"
#include "bounds.h"
#include "compress.h"

namespace vc {

namespace {

__device__ __forceinline__ float load_elem(const void* p, int64_t i, int dtype) {
  return dtype == VC_BF16 ? bf2f(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}
__device__ __forceinline__ uint16_t f2h_bits(float f) { return bitcast<uint16_t>((_Float16)f); }
__device__ __forceinline__ float h2f_bits(uint16_t h) { return float(bitcast<_Float16>(h)); }

__device__ __forceinline__ void scale_zero(float mn, float mx, int bits, uint16_t& sh, uint16_t& zh) {
  const float range = __fsub_rn(mx, mn);
  const float sc = __fdiv_rn(range, float((1 << bits) - 1));
  sh = f2h_bits(sc);
  zh = f2h_bits(mn);
}
__device__ __forceinline__ uint32_t quant_code(float x, float z, float s, int bits) {
  if (s == 0.f) return 0u;
  float t = rintf(__fdiv_rn(__fsub_rn(x, z), s));
  t = fminf(fmaxf(t, 0.f), float((1 << bits) - 1));
  return uint32_t(t);
}

// K scale/zero: one thread per (layer*head, group, channel); reads G tokens of one channel.
__global__ void k_scales_kernel(const void* k, int dtype, int src_cap, int D, int group, int ng, int bits, int n_lh,
                                uint16_t* ks, uint16_t* kz) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(n_lh) * ng * D;
  if (i >= total) return;
  const int d = int(i % D);
  const int g = int((i / D) % ng);
  const int lh = int(i / (int64_t(D) * ng));
  const int64_t base = int64_t(lh) * src_cap * D;
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
  for (int t = 0; t < group; t++) {
    const float x = load_elem(k, base + int64_t(g * group + t) * D + d, dtype);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  uint16_t sh, zh;
  scale_zero(mn, mx, bits, sh, zh);
  ks[i] = sh;
  kz[i] = zh;
}

// V scale/zero: one thread per (layer*head, token, channel group); reads G channels of one token.
__global__ void v_scales_kernel(const void* v, int dtype, int src_cap, int D, int group, int tq, int bits, int n_lh,
                                uint16_t* vs, uint16_t* vz) {
  const int nh = D / group;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(n_lh) * tq * nh;
  if (i >= total) return;
  const int h = int(i % nh);
  const int t = int((i / nh) % tq);
  const int lh = int(i / (int64_t(nh) * tq));
  const int64_t base = (int64_t(lh) * src_cap + t) * D + h * group;
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
  for (int c = 0; c < group; c++) {
    const float x = load_elem(v, base + c, dtype);
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  uint16_t sh, zh;
  scale_zero(mn, mx, bits, sh, zh);
  vs[i] = sh;
  vz[i] = zh;
}

// K codes: one thread per 32-bit word of a token row (D*b/32 words per row).
__global__ void k_codes_kernel(const void* k, int dtype, int src_cap, int D, int group, int ng, int tq, int bits,
                               int n_lh, const uint16_t* ks, const uint16_t* kz, uint32_t* kc) {
  const int words = D * bits / 32;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(n_lh) * tq * words;
  if (i >= total) return;
  const int w = int(i % words);
  const int t = int((i / words) % tq);
  const int lh = int(i / (int64_t(words) * tq));
  const int g = t / group;
  const int64_t xbase = (int64_t(lh) * src_cap + t) * D;
  const int64_t sbase = (int64_t(lh) * ng + g) * D;
  uint32_t out = 0;
  const int c0 = (32 * w) / bits, c1 = (32 * w + 31) / bits;
  for (int c = c0; c <= c1 && c < D; c++) {
    const uint32_t code =
        quant_code(load_elem(k, xbase + c, dtype), h2f_bits(kz[sbase + c]), h2f_bits(ks[sbase + c]), bits);
    const int bit = c * bits - 32 * w;  // may be negative for a code straddling into this word
    if (bit >= 0) out |= code << bit;
    else out |= code >> (-bit);
  }
  kc[i] = out;
}

// V codes: per (layer*head, 64-token block, channel), 2*b words; token i of the block at bits [i*b, i*b+b).
__global__ void v_codes_kernel(const void* v, int dtype, int src_cap, int D, int group, int tq, int bits, int n_lh,
                               const uint16_t* vs, const uint16_t* vz, uint32_t* vcode) {
  const int words = 2 * bits;
  const int nblk = tq / 64;
  const int nh = D / group;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(n_lh) * nblk * D * words;
  if (i >= total) return;
  const int w = int(i % words);
  const int d = int((i / words) % D);
  const int blk = int((i / (int64_t(words) * D)) % nblk);
  const int lh = int(i / (int64_t(words) * D * nblk));
  const int h = d / group;
  uint32_t out = 0;
  const int c0 = (32 * w) / bits, c1 = (32 * w + 31) / bits;
  for (int c = c0; c <= c1 && c < 64; c++) {
    const int t = blk * 64 + c;
    const int64_t si = (int64_t(lh) * tq + t) * nh + h;
    const uint32_t code =
        quant_code(load_elem(v, (int64_t(lh) * src_cap + t) * D + d, dtype), h2f_bits(vz[si]), h2f_bits(vs[si]), bits);
    const int bit = c * bits - 32 * w;
    if (bit >= 0) out |= code << bit;
    else out |= code >> (-bit);
  }
  vcode[i] = out;
}

// Copy rows [r0, r0 + nrows) of every (layer, head) from a [n_lh][src_cap][D] buffer into a dense [n_lh][nrows][D].
__global__ void copy_rows_kernel(const uint8_t* src, int src_cap, int r0, int nrows, int row_bytes, int n_lh,
                                 uint8_t* dst) {
  const int64_t words = int64_t(row_bytes) / 4;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(n_lh) * nrows * words;
  if (i >= total) return;
  const int64_t w = i % words;
  const int r = int((i / words) % nrows);
  const int lh = int(i / (words * nrows));
  reinterpret_cast<uint32_t*>(dst)[i] =
      reinterpret_cast<const uint32_t*>(src + (int64_t(lh) * src_cap + r0 + r) * row_bytes)[w];
}

// ---------------------------------------------------------------- token drop
// Softmax statistics (M, L) of every observation query from split partials.
__global__ void merge_ml_kernel(const float* part, int n_rows_heads, int s_used, int s_total, int D, float* ml) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_rows_heads) return;
  const float* p = part + int64_t(i) * s_total * (D + 2);
  float M = NEG_INF;
  for (int s = 0; s < s_used; s++) M = fmaxf(M, p[s * (D + 2)]);
  float L = 0.f;
  for (int s = 0; s < s_used; s++) {
    const float ms = p[s * (D + 2)];
    L = fmaf(p[s * (D + 2) + 1], ms == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(ms - M), L);
  }
  ml[2 * i] = M;
  ml[2 * i + 1] = L;
}

// score[t] = mean over (h in group, w < W) of 2^(q.k_t * sl2 - M) / L for candidate t < n_cand.
// One workgroup of 256 threads per (layer*head, 64 candidates): thread (t = tid%64, part = tid/64)
// sums a quarter of the query rows; parts are merged in fixed order.
__global__ __launch_bounds__(256) void tokdrop_scores_kernel(const void* k, const void* q_obs, const float* ml, int dtype,
                                                             int src_cap, int D, int Hq, int Hkv, int W, int n_cand,
                                                             float sl2, float* scores) {
  __shared__ float qs[128][129];
  __shared__ float acc[4][64];
  const int G = Hq / Hkv;
  const int lh = blockIdx.y;
  const int l = lh / Hkv, j = lh % Hkv;
  const int tid = threadIdx.x;
  const int t = blockIdx.x * 64 + (tid & 63);
  const int part = tid >> 6;
  const int n_q = G * W;
  float sum = 0.f;
  // query rows r = h*W + w (h within the group), processed 128 at a time (D <= 128)
  for (int r0 = 0; r0 < n_q; r0 += 128) {
    const int nr = min(128, n_q - r0);
    __syncthreads();
    for (int e = tid; e < nr * D; e += 256) {
      const int r = r0 + e / D, d = e % D;
      const int h = r / W, w = r % W;
      qs[e / D][d] = load_elem(q_obs, ((int64_t(l) * W + w) * Hq + j * G + h) * D + d, dtype);
    }
    __syncthreads();
    if (t < n_cand) {
      const int64_t kb = (int64_t(lh) * src_cap + t) * D;
      for (int rr = part; rr < nr; rr += 4) {
        float dot = 0.f;
        for (int d = 0; d < D; d++) dot = fmaf(qs[rr][d], load_elem(k, kb + d, dtype), dot);
        const int r = r0 + rr;
        const int h = r / W, w = r % W;
        const int64_t mi = ((int64_t(l) * W + w) * Hq + j * G + h) * 2;
        sum += __builtin_amdgcn_exp2f(dot * sl2 - ml[mi]) / ml[mi + 1];
      }
    }
  }
  acc[part][tid & 63] = sum;
  __syncthreads();
  if (part == 0 && t < n_cand) {
    const float s = ((acc[0][tid] + acc[1][tid]) + acc[2][tid]) + acc[3][tid];
    scores[int64_t(lh) * n_cand + t] = s / float(n_q);
  }
}

// The same scores for bf16 caches with head_dim 128, on MFMAs.  Workgroup = 4 waves =
// (layer*head, 256 candidates); wave w takes candidates 64w .. 64w + 63 of the chunk as four
// 16-key sub-tiles.  Per 16-row block of the observation rows (staged in LDS, 128 at a time)
// S = Q K^T runs as 16x16x32 bf16 MFMAs: A = Q rows from LDS, B = K^T fragments held in
// registers for the whole kernel (lane l: candidate l % 16 of each sub-tile, channels
// 8 (l / 16) .. + 8 of each 32-channel chunk), read straight from HBM once.  Lane l then holds
// the scores of rows 4 (l / 16) + jj of the block for its candidate; it adds
// 2^(s sl2 - M_row) / L_row over its rows (1 / L_row taken once per row), and the four lane
// groups are added in fixed order.
constexpr int SC_ROWS = 128;            // observation rows staged per pass
constexpr int SC_PITCH = 128 + 8;       // bf16 per staged row (pad breaks bank aliasing)

__global__ __launch_bounds__(256) void tokdrop_scores_bf16_kernel(const uint16_t* k, const uint16_t* q_obs,
                                                                  const float* ml, int src_cap, int Hq, int Hkv,
                                                                  int W, int n_cand, float sl2, float* scores) {
  __shared__ __attribute__((aligned(16))) uint16_t qs[SC_ROWS * SC_PITCH];
  __shared__ float2 mls[SC_ROWS];  // (-M, 1 / L) per staged row
  constexpr int D = 128;
  const int G = Hq / Hkv;
  const int lh = blockIdx.y;
  const int l = lh / Hkv, j = lh % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, g = lane >> 4;
  const int n_q = G * W;
  const int t_base = blockIdx.x * 256 + 64 * wave;
  u32x4 kf[4][4];
#pragma unroll
  for (int kt = 0; kt < 4; kt++) {
    const int t = t_base + 16 * kt + r16;
    const uint16_t* kp = k + (int64_t(lh) * src_cap + (t < n_cand ? t : 0)) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < 4; c++) kf[kt][c] = t < n_cand ? ld_nt(kp + 32 * c) : u32x4{0, 0, 0, 0};
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < n_q; r0 += SC_ROWS) {
    const int nr = min(SC_ROWS, n_q - r0);
    __syncthreads();
    for (int e = tid; e < SC_ROWS * 16; e += 256) {
      const int rr = e >> 4, ch = e & 15;
      u32x4 x = u32x4{0, 0, 0, 0};
      if (rr < nr) {
        const int r = r0 + rr, h = r / W, w = r % W;
        x = *reinterpret_cast<const u32x4*>(q_obs + ((int64_t(l) * W + w) * Hq + j * G + h) * D + 8 * ch);
      }
      *reinterpret_cast<u32x4*>(qs + rr * SC_PITCH + 8 * ch) = x;
    }
    for (int rr = tid; rr < SC_ROWS; rr += 256) {
      float2 m = float2{NEG_INF, 0.f};  // padding rows add exp2(-inf) * 0 = 0
      if (rr < nr) {
        const int r = r0 + rr, h = r / W, w = r % W;
        const int64_t mi = ((int64_t(l) * W + w) * Hq + j * G + h) * 2;
        m = float2{-ml[mi], 1.f / ml[mi + 1]};
      }
      mls[rr] = m;
    }
    __syncthreads();
    const int nb = (nr + 15) >> 4;
    for (int rb = 0; rb < nb; rb++) {
      u32x4 qa[4];
#pragma unroll
      for (int c = 0; c < 4; c++) qa[c] = *reinterpret_cast<const u32x4*>(qs + (16 * rb + r16) * SC_PITCH + 32 * c + 8 * g);
      float2 m[4];
#pragma unroll
      for (int jj = 0; jj < 4; jj++) m[jj] = mls[16 * rb + 4 * g + jj];
#pragma unroll
      for (int kt = 0; kt < 4; kt++) {
        f32x4 sv = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; c++) sv = mfma_bf16(qa[c], kf[kt][c], sv);
#pragma unroll
        for (int jj = 0; jj < 4; jj++) acc[kt] += __builtin_amdgcn_exp2f(fmaf(sv[jj], sl2, m[jj].x)) * m[jj].y;
      }
    }
  }
#pragma unroll
  for (int kt = 0; kt < 4; kt++) {
    acc[kt] += shfl_xor(acc[kt], 16);
    acc[kt] += shfl_xor(acc[kt], 32);
    const int t = t_base + 16 * kt + r16;
    if (g == 0 && t < n_cand) scores[int64_t(lh) * n_cand + t] = acc[kt] / float(n_q);
  }
}

// Deterministic top-k per (layer*head): radix select on the float bits (scores are >= 0, so the
// unsigned bit pattern orders them), ties resolved towards the smaller index; output ascending.
constexpr int SEL_THREADS = 1024;

__global__ __launch_bounds__(SEL_THREADS) void topk_select_kernel(const float* scores, int n_cand, int n_top,
                                                                  int n_recent, int kk, int32_t* idx) {
  __shared__ int hist[256];
  __shared__ int s_digit, s_k;
  __shared__ int chunk_count[SEL_THREADS];
  const int lh = blockIdx.x;
  const int tid = threadIdx.x;
  const uint32_t* sb = reinterpret_cast<const uint32_t*>(scores + int64_t(lh) * n_cand);
  int32_t* out = idx + int64_t(lh) * kk;
  uint32_t prefix = 0, pmask = 0;
  int k = n_top;
  for (int pass = 0; pass < 4; pass++) {
    const int shift = 24 - 8 * pass;
    for (int b = tid; b < 256; b += SEL_THREADS) hist[b] = 0;
    __syncthreads();
    for (int t = tid; t < n_cand; t += SEL_THREADS) {
      const uint32_t v = sb[t];
      if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int acc = 0, d = 255;
      for (; d > 0; d--) {
        if (acc + hist[d] >= k) break;
        acc += hist[d];
      }
      s_digit = d;
      s_k = k - acc;
    }
    __syncthreads();
    prefix |= uint32_t(s_digit) << shift;
    pmask |= 255u << shift;
    k = s_k;
    __syncthreads();
  }
  const uint32_t thr = prefix;  // the n_top-th largest value; take all > thr and the first k equal to thr
  const int k_eq = k;
  // contiguous chunks per thread keep the output ascending after a prefix sum
  const int per = (n_cand + SEL_THREADS - 1) / SEL_THREADS;
  const int lo = tid * per, hi = min(n_cand, lo + per);
  int n_gt = 0, n_eq = 0;
  for (int t = lo; t < hi; t++) {
    const uint32_t v = sb[t];
    n_gt += v > thr;
    n_eq += v == thr;
  }
  // exclusive prefix of equal counts -> how many equals precede this chunk
  chunk_count[tid] = n_eq;
  __syncthreads();
  for (int off = 1; off < SEL_THREADS; off <<= 1) {
    const int x = tid >= off ? chunk_count[tid - off] : 0;
    __syncthreads();
    chunk_count[tid] += x;
    __syncthreads();
  }
  const int eq_before = chunk_count[tid] - n_eq;
  const int take_eq = max(0, min(n_eq, k_eq - eq_before));
  const int sel = n_gt + take_eq;
  __syncthreads();
  chunk_count[tid] = sel;
  __syncthreads();
  for (int off = 1; off < SEL_THREADS; off <<= 1) {
    const int x = tid >= off ? chunk_count[tid - off] : 0;
    __syncthreads();
    chunk_count[tid] += x;
    __syncthreads();
  }
  int o = chunk_count[tid] - sel;
  int eq_seen = 0;
  for (int t = lo; t < hi; t++) {
    const uint32_t v = sb[t];
    bool take = v > thr;
    if (v == thr) {
      take = eq_seen < take_eq;
      eq_seen++;
    }
    if (take && o < n_top) out[o++] = t;
  }
  // recent window
  for (int r = tid; r < n_recent; r += SEL_THREADS) out[n_top + r] = n_cand + r;
}

__global__ void iota_kernel(int32_t* idx, int n_lh, int kk) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(n_lh) * kk) return;
  idx[i] = int32_t(i % kk);
}

// Gather kept rows: dst[lh][r] = src[lh][idx[lh][r]] (row_bytes each).
__global__ void gather_rows_kernel(const uint8_t* src, int src_cap, int row_bytes, const int32_t* idx, int kk, int n_lh,
                                   uint8_t* dst) {
  const int64_t words = row_bytes / 4;
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(n_lh) * kk * words) return;
  const int64_t w = i % words;
  const int r = int((i / words) % kk);
  const int lh = int(i / (words * kk));
  const int t = idx[int64_t(lh) * kk + r];
  if (t < 0 || t >= src_cap) {  // never for a valid selection; keeps a bad index from reading out of bounds
    reinterpret_cast<uint32_t*>(dst)[i] = 0u;
    return;
  }
  reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(src + (int64_t(lh) * src_cap + t) * row_bytes)[w];
}

// Per (layer*head, 64-position tile): bit o of mask = position 64*tile + o is kept;
// cnt = kept positions before the tile (idx is ascending, so a binary search finds it).
// Key-norm ranking: thread t of layer blockIdx.y sums k^2 over the channels of each KV head
// in order, takes the square root and averages over the heads in order; the score is written
// to every head's row so that each head's selection is the layer's one.
__global__ void keynorm_scores_kernel(const void* k, int dtype, int src_cap, int D, int Hkv, int n_cand,
                                      float* scores) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int l = blockIdx.y;
  if (t >= n_cand) return;
  float e = 0.f;
  for (int j = 0; j < Hkv; j++) {
    const int64_t base = (int64_t(l * Hkv + j) * src_cap + t) * D;
    float ss = 0.f;
    for (int d = 0; d < D; d++) {
      const float x = load_elem(k, base + d, dtype);
      ss = __fmaf_rn(x, x, ss);
    }
    e += __fsqrt_rn(ss);
  }
  e = __fdiv_rn(e, float(Hkv));
  for (int j = 0; j < Hkv; j++) scores[int64_t(l * Hkv + j) * n_cand + t] = e;
}

__global__ void keep_tiles_kernel(const int32_t* idx, int kk, int n_lh, int n_tiles, uint64_t* mask, int32_t* cnt) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= int64_t(n_lh) * n_tiles) return;
  const int lh = int(i / n_tiles), tile = int(i % n_tiles);
  const int32_t* id = idx + int64_t(lh) * kk;
  const int t0 = tile * 64;
  int lo = 0, hi = kk;  // first r with id[r] >= t0
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (id[mid] < t0) lo = mid + 1;
    else hi = mid;
  }
  uint64_t m = 0;
  for (int r = lo; r < kk && id[r] < t0 + 64; r++) m |= uint64_t(1) << (id[r] - t0);
  mask[i] = m;
  cnt[i] = lo;
}

// Rows of [L*Hkv][src_cap] positions [0, T) that were not kept, compacted in position
// order into dst [L*Hkv][dst_cap] (row_bytes each), for layers' heads [lh0, lh0 + n_lh).
__global__ void gather_dropped_kernel(const uint8_t* src, int src_cap, int T, int row_bytes, const uint64_t* mask,
                                      const int32_t* cnt, int n_tiles, int lh0, uint8_t* dst, int dst_cap) {
  const int lh = lh0 + blockIdx.y;
  const int t = blockIdx.x;  // position
  if (t >= T) return;
  const int tile = t >> 6, o = t & 63;
  const uint64_t m = mask[int64_t(lh) * n_tiles + tile];
  if ((m >> o) & 1) return;
  const int below = __popcll(m & ((uint64_t(1) << o) - 1));
  const int r = t - cnt[int64_t(lh) * n_tiles + tile] - below;
  if (r < 0 || r >= dst_cap) return;  // never for a consistent (idx, mask, cnt)
  const uint32_t* sp = reinterpret_cast<const uint32_t*>(src + (int64_t(lh) * src_cap + t) * row_bytes);
  uint32_t* dp = reinterpret_cast<uint32_t*>(dst + (int64_t(blockIdx.y) * dst_cap + r) * row_bytes);
  for (int w = threadIdx.x; w < row_bytes / 4; w += blockDim.x) dp[w] = sp[w];
}

}  // namespace

vc_status compress_layout(const vc_compress_desc* d, vc_compress_layout* L) {
  VC_REQUIRE(d != nullptr && L != nullptr, VC_ERR_ARG, "compress: null descriptor");
  VC_REQUIRE(d->n_layers > 0 && d->n_kv_heads > 0 && d->n_q_heads % d->n_kv_heads == 0 && d->seq_len > 0 &&
                 d->src_cap >= d->seq_len,
             VC_ERR_ARG, "compress: bad shape");
  VC_REQUIRE(d->dtype == VC_F32 || d->dtype == VC_BF16, VC_ERR_ARG, "compress: bad dtype");
  const int64_t LH = int64_t(d->n_layers) * d->n_kv_heads;
  const int64_t D = d->head_dim, T = d->seq_len;
  const int64_t eb = d->dtype == VC_BF16 ? 2 : 4;
  *L = vc_compress_layout{};
  size_t off = 0;
  auto sect = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  if (d->kind == VC_TOKDROP) {
    VC_REQUIRE(d->score == VC_SCORE_ATTN || d->score == VC_SCORE_KEYNORM, VC_ERR_ARG, "tokdrop: bad score %d",
               d->score);
    VC_REQUIRE(d->keep_recent >= 0 && d->keep_total > 0 && (d->obs_window > 0 || d->score == VC_SCORE_KEYNORM),
               VC_ERR_ARG, "tokdrop: bad knobs");
    const int64_t nrec = std::min<int64_t>(d->keep_recent, T);
    const int64_t kk = std::min<int64_t>(T, std::max<int64_t>(d->keep_total, nrec));
    L->n_main = int32_t(kk);
    L->n_resid = 0;
    L->n_tiles = int32_t(cdiv(T, 64));
    L->n_host = int32_t(T - kk);
    L->k_main = sect(LH * kk * D * eb);
    L->v_main = sect(LH * kk * D * eb);
    L->idx = sect(LH * kk * 4);
    L->keep_mask = sect(LH * L->n_tiles * 8);
    L->keep_cnt = sect(LH * L->n_tiles * 4);
  } else if (d->kind == VC_QUANT) {
    VC_REQUIRE(d->bits >= 2 && d->bits <= 4, VC_ERR_UNSUPPORTED, "quant: bits must be 2, 3 or 4");
    VC_REQUIRE(d->group == 64 || d->group == 128, VC_ERR_UNSUPPORTED, "quant: group must be 64 or 128");
    VC_REQUIRE(D == 128, VC_ERR_UNSUPPORTED, "quant: head_dim must be 128");
    const int64_t tq = T / d->group * d->group;
    const int64_t ng = tq / d->group;
    L->n_main = int32_t(tq);
    L->n_resid = int32_t(T - tq);
    L->n_host = int32_t(T);
    L->kc = sect(LH * tq * D * d->bits / 8);
    L->vc = sect(LH * tq * D * d->bits / 8);
    L->ks = sect(LH * ng * D * 2);
    L->kz = sect(LH * ng * D * 2);
    L->vs = sect(LH * tq * (D / d->group) * 2);
    L->vz = sect(LH * tq * (D / d->group) * 2);
    L->kr = sect(LH * (T - tq) * D * eb);
    L->vr = sect(LH * (T - tq) * D * eb);
  } else {
    VC_REQUIRE(false, VC_ERR_ARG, "compress: unknown kind %d", d->kind);
  }
  L->total = off;
  return VC_OK;
}

vc_status compress_ws_bytes(const vc_compress_desc* d, size_t* ws) {
  *ws = 0;
  if (d->kind != VC_TOKDROP) return VC_OK;
  const int64_t LH = int64_t(d->n_layers) * d->n_kv_heads;
  const int64_t T = d->seq_len, D = d->head_dim;
  if (d->score == VC_SCORE_KEYNORM) {
    *ws = align256(LH * T * 4);  // scores only
    return VC_OK;
  }
  const int64_t W = std::min<int64_t>(d->obs_window, T);
  const int64_t split = 1024;
  const int64_t S = cdiv(T, split);
  const int64_t rows_heads = int64_t(d->n_layers) * W * d->n_q_heads;
  size_t b = 0;
  b += align256(rows_heads * S * (D + 2) * 4);  // partials
  b += align256(rows_heads * 2 * 4);            // (M, L)
  b += align256(LH * T * 4);                    // scores
  *ws = b;
  return VC_OK;
}

vc_status compress_run(const vc_compress_desc* d, const void* k, const void* v, const void* q_obs, void* out,
                       size_t out_bytes, void* ws, size_t ws_bytes, hipStream_t s) {
  vc_compress_layout L;
  vc_status st = compress_layout(d, &L);
  if (st) return st;
  VC_REQUIRE(k != nullptr && v != nullptr && out != nullptr, VC_ERR_ARG, "vc_compress: null pointer");
  VC_REQUIRE(out_bytes >= L.total, VC_ERR_CAPACITY, "vc_compress: output %zu < %zu bytes", out_bytes, L.total);
  const int n_lh = d->n_layers * d->n_kv_heads;
  const int D = d->head_dim, T = d->seq_len;
  const int eb = d->dtype == VC_BF16 ? 2 : 4;
  uint8_t* o = static_cast<uint8_t*>(out);
  if (dbg_on()) {
    // prompt rows [0, T) of every (layer, head), the blob, and (token drop) the observation
    // queries and the workspace; the observation attention checks its own launch below
    const int64_t row = int64_t(D) * eb, pitch = int64_t(d->src_cap) * row;
    size_t need = 0;
    compress_ws_bytes(d, &need);
    const bool obs = d->kind == VC_TOKDROP && d->score == VC_SCORE_ATTN;
    const int64_t W = std::min(d->obs_window, T);
    if (vc_status st = dbg_check("compress", {dbg_2d("prompt K", k, pitch, T * row, n_lh),
                                              dbg_2d("prompt V", v, pitch, T * row, n_lh),
                                              {"blob", out, int64_t(L.total)},
                                              {"workspace", ws, int64_t(need)},
                                              {"observation queries", q_obs,
                                               obs ? int64_t(d->n_layers) * W * d->n_q_heads * row : 0}}))
      return st;
  }
  if (dbg_dry() && !(d->kind == VC_TOKDROP && d->score == VC_SCORE_ATTN && L.n_main - std::min(d->keep_recent, T) <
                                                                              T - std::min(d->keep_recent, T)))
    return VC_OK;
  if (d->kind == VC_QUANT) {
    const int tq = L.n_main, ng = tq / d->group, b = d->bits;
    uint16_t* ks = reinterpret_cast<uint16_t*>(o + L.ks);
    uint16_t* kz = reinterpret_cast<uint16_t*>(o + L.kz);
    uint16_t* vs = reinterpret_cast<uint16_t*>(o + L.vs);
    uint16_t* vz = reinterpret_cast<uint16_t*>(o + L.vz);
    if (tq > 0) {
      int64_t n = int64_t(n_lh) * ng * D;
      hipLaunchKernelGGL(k_scales_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, k, d->dtype, d->src_cap, D, d->group,
                         ng, b, n_lh, ks, kz);
      n = int64_t(n_lh) * tq * (D / d->group);
      hipLaunchKernelGGL(v_scales_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, v, d->dtype, d->src_cap, D, d->group,
                         tq, b, n_lh, vs, vz);
      n = int64_t(n_lh) * tq * (D * b / 32);
      hipLaunchKernelGGL(k_codes_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, k, d->dtype, d->src_cap, D, d->group,
                         ng, tq, b, n_lh, ks, kz, reinterpret_cast<uint32_t*>(o + L.kc));
      n = int64_t(n_lh) * (tq / 64) * D * 2 * b;
      hipLaunchKernelGGL(v_codes_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, v, d->dtype, d->src_cap, D, d->group,
                         tq, b, n_lh, vs, vz, reinterpret_cast<uint32_t*>(o + L.vc));
      VC_LAUNCH_CHECK();
    }
    if (L.n_resid > 0) {
      const int64_t n = int64_t(n_lh) * L.n_resid * (D * eb / 4);
      hipLaunchKernelGGL(copy_rows_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, static_cast<const uint8_t*>(k),
                         d->src_cap, tq, L.n_resid, D * eb, n_lh, o + L.kr);
      hipLaunchKernelGGL(copy_rows_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, static_cast<const uint8_t*>(v),
                         d->src_cap, tq, L.n_resid, D * eb, n_lh, o + L.vr);
      VC_LAUNCH_CHECK();
    }
    return VC_OK;
  }
  // ---- token drop
  size_t need = 0;
  compress_ws_bytes(d, &need);
  const int kk = L.n_main;
  const int n_recent = std::min(d->keep_recent, T);
  const int n_cand = T - n_recent;
  const int n_top = kk - n_recent;
  int32_t* idx = reinterpret_cast<int32_t*>(o + L.idx);
  if (n_top >= n_cand) {
    // everything fits: keep all rows
    const int64_t n = int64_t(n_lh) * kk;
    hipLaunchKernelGGL(iota_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, idx, n_lh, kk);
    VC_LAUNCH_CHECK();
  } else if (d->score == VC_SCORE_KEYNORM) {
    VC_REQUIRE(ws != nullptr && ws_bytes >= need, VC_ERR_CAPACITY, "vc_compress: workspace %zu < %zu", ws_bytes, need);
    float* scores = static_cast<float*>(ws);
    hipLaunchKernelGGL(keynorm_scores_kernel, dim3(cdiv(n_cand, 256), d->n_layers), dim3(256), 0, s, k, d->dtype,
                       d->src_cap, D, d->n_kv_heads, n_cand, scores);
    VC_LAUNCH_CHECK();
    hipLaunchKernelGGL(topk_select_kernel, dim3(n_lh), dim3(SEL_THREADS), 0, s, scores, n_cand, n_top, n_recent, kk,
                       idx);
    VC_LAUNCH_CHECK();
  } else {
    VC_REQUIRE(q_obs != nullptr, VC_ERR_ARG, "vc_compress: token drop needs q_obs");
    VC_REQUIRE(ws != nullptr && ws_bytes >= need, VC_ERR_CAPACITY, "vc_compress: workspace %zu < %zu", ws_bytes, need);
    VC_REQUIRE(D <= 128, VC_ERR_UNSUPPORTED, "tokdrop: head_dim > 128");
    const int W = std::min(d->obs_window, T);
    const int G = d->n_q_heads / d->n_kv_heads;
    const int split = 1024;
    const int S = int(cdiv(T, split));
    const int64_t rows_heads = int64_t(W) * d->n_q_heads;  // per layer
    uint8_t* w8 = static_cast<uint8_t*>(ws);
    float* part = reinterpret_cast<float*>(w8);
    float* ml = reinterpret_cast<float*>(w8 + align256(int64_t(d->n_layers) * rows_heads * S * (D + 2) * 4));
    float* scores = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ml) +
                                             align256(int64_t(d->n_layers) * rows_heads * 2 * 4));
    const float sl2 = LOG2E / sqrtf(float(D));
    // pass 1: softmax statistics of the observation queries (one layer at a time through attention)
    for (int l = 0; l < d->n_layers; l++) {
      AttnArgs a{};
      a.n_req = 1;
      a.Hq = d->n_q_heads;
      a.Hkv = d->n_kv_heads;
      a.G = G;
      a.split_len = split;
      a.head_dim = D;
      a.scale_log2 = sl2;
      a.n_rowblocks = int(cdiv(int64_t(W) * G, ATT_RB));
      a.max_splits = S;
      AttnReq& r = a.r[0];
      const int64_t lstride = int64_t(d->n_kv_heads) * d->src_cap * D * eb;
      r.q = static_cast<const uint8_t*>(q_obs) + int64_t(l) * W * d->n_q_heads * D * eb;
      r.a = KVSeg{static_cast<const uint8_t*>(k) + l * lstride, static_cast<const uint8_t*>(v) + l * lstride,
                  int64_t(d->src_cap) * D, T, 0};
      r.b = KVSeg{nullptr, nullptr, 0, 0, 0};
      r.part = part + int64_t(l) * rows_heads * S * (D + 2);
      r.n_rows = W;
      r.lim0 = T - W;
      r.s_off = 0;
      r.s_total = S;
      r.n_splits = S;
      st = launch_attn(a, d->dtype, s);
      if (st) return st;
    }
    if (dbg_dry()) return VC_OK;
    {
      const int n = int(int64_t(d->n_layers) * rows_heads);
      hipLaunchKernelGGL(merge_ml_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, part, n, S, S, D, ml);
      VC_LAUNCH_CHECK();
    }
    // pass 2: scores of the candidates
    if (d->dtype == VC_BF16 && D == 128) {
      hipLaunchKernelGGL(tokdrop_scores_bf16_kernel, dim3(cdiv(n_cand, 256), n_lh), dim3(256), 0, s,
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(q_obs), ml, d->src_cap,
                         d->n_q_heads, d->n_kv_heads, W, n_cand, sl2, scores);
    } else {
      hipLaunchKernelGGL(tokdrop_scores_kernel, dim3(cdiv(n_cand, 64), n_lh), dim3(256), 0, s, k, q_obs, ml, d->dtype,
                         d->src_cap, D, d->n_q_heads, d->n_kv_heads, W, n_cand, sl2, scores);
    }
    VC_LAUNCH_CHECK();
    hipLaunchKernelGGL(topk_select_kernel, dim3(n_lh), dim3(SEL_THREADS), 0, s, scores, n_cand, n_top, n_recent, kk,
                       idx);
    VC_LAUNCH_CHECK();
  }
  {
    const int64_t n = int64_t(n_lh) * kk * (D * eb / 4);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, static_cast<const uint8_t*>(k),
                       d->src_cap, D * eb, idx, kk, n_lh, o + L.k_main);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, static_cast<const uint8_t*>(v),
                       d->src_cap, D * eb, idx, kk, n_lh, o + L.v_main);
    VC_LAUNCH_CHECK();
  }
  {
    const int64_t n = int64_t(n_lh) * L.n_tiles;
    hipLaunchKernelGGL(keep_tiles_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, idx, kk, n_lh, L.n_tiles,
                       reinterpret_cast<uint64_t*>(o + L.keep_mask), reinterpret_cast<int32_t*>(o + L.keep_cnt));
    VC_LAUNCH_CHECK();
  }
  return VC_OK;
}

vc_status gather_dropped(const vc_compress_desc* d, const void* comp, const void* src, int src_cap, int lh0, int n_lh,
                         void* dst, int dst_cap, hipStream_t s) {
  vc_compress_layout L;
  vc_status st = compress_layout(d, &L);
  if (st) return st;
  VC_REQUIRE(d->kind == VC_TOKDROP, VC_ERR_ARG, "gather_dropped: not a token-drop cache");
  VC_REQUIRE(lh0 >= 0 && n_lh > 0 && lh0 + n_lh <= d->n_layers * d->n_kv_heads && dst_cap >= L.n_host &&
                 src_cap >= d->seq_len,
             VC_ERR_ARG, "gather_dropped: bad range");
  if (L.n_host == 0) return VC_OK;
  const int eb = d->dtype == VC_BF16 ? 2 : 4;
  const uint8_t* o = static_cast<const uint8_t*>(comp);
  {
    const int64_t row = int64_t(d->head_dim) * eb, nt = L.n_tiles;
    const int64_t lh_all = int64_t(d->n_layers) * d->n_kv_heads;
    VC_DBG_LAUNCH("gather_dropped",
                  dbg_2d("prompt rows", static_cast<const uint8_t*>(src) + lh0 * int64_t(src_cap) * row,
                         int64_t(src_cap) * row, d->seq_len * row, n_lh),
                  dbg_2d("dropped rows", dst, int64_t(dst_cap) * row, int64_t(dst_cap) * row, n_lh),
                  {"kept-tile masks", o + L.keep_mask, lh_all * nt * 8}, {"kept-tile counts", o + L.keep_cnt, lh_all * nt * 4});
  }
  hipLaunchKernelGGL(gather_dropped_kernel, dim3(d->seq_len, n_lh), dim3(64), 0, s, static_cast<const uint8_t*>(src),
                     src_cap, d->seq_len, d->head_dim * eb, reinterpret_cast<const uint64_t*>(o + L.keep_mask),
                     reinterpret_cast<const int32_t*>(o + L.keep_cnt), L.n_tiles, lh0, static_cast<uint8_t*>(dst),
                     dst_cap);
  VC_LAUNCH_CHECK();
  return VC_OK;
}

}  // namespace vc
