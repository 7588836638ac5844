// Row-wise kernels of the forward pass and the accept / commit steps.
#include "bounds.h"
#include "elementwise.h"

namespace vc {

namespace {

__device__ __forceinline__ float ld(const void* p, int64_t i, int dt) {
  return dt == VC_BF16 ? bf2f(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}
__device__ __forceinline__ void st(void* p, int64_t i, float v, int dt) {
  if (dt == VC_BF16) static_cast<uint16_t*>(p)[i] = f2bf(v);
  else static_cast<float*>(p)[i] = v;
}

// Row r of h = row tok[r] of E.  A token outside [0, V) (the -1 that argmax writes for a row with
// no finite logit, or any other invalid id) reads nothing: its row becomes quiet NaN, which the
// rest of the forward carries into that row's logits and so into another -1.
__global__ void embed_kernel(const void* E, const int32_t* tok, void* h, int d, int V, int dt) {
  const int r = blockIdx.y;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= d) return;
  const int64_t t = tok[r];
  const int64_t o = int64_t(r) * d + c;
  if (t < 0 || t >= V) {  // the table is not touched
    if (dt == VC_BF16) static_cast<uint16_t*>(h)[o] = uint16_t(0x7fc0);
    else static_cast<float*>(h)[o] = __builtin_nanf("");
    return;
  }
  if (dt == VC_BF16) static_cast<uint16_t*>(h)[o] = static_cast<const uint16_t*>(E)[t * d + c];
  else static_cast<float*>(h)[o] = static_cast<const float*>(E)[t * d + c];
}

// y = x / sqrt(mean(x^2) + eps) * g, one workgroup of 256 threads per row.  bf16 rows with
// d a multiple of 2048 (up to 8192): every thread holds its 16-byte chunks c = tid + 256 i in
// registers, so the row is read once; the sum of squares is reduced in a fixed order (each
// thread's chunks in order, then a butterfly within each wave, then the four waves in order),
// identically for every row.  Other rows: the same reduction over single elements.
constexpr int RMS_MAXC = 4;  // 16-byte chunks per thread (d <= 8192)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* x, const void* g, void* y, int d, float eps, int dt) {
  __shared__ float red[4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = int64_t(r) * d;
  const bool vec = dt == VC_BF16 && d % 2048 == 0 && d <= 2048 * RMS_MAXC;  // uniform
  float ss = 0.f;
  u32x4 xv[RMS_MAXC];
  if (vec) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + base);
#pragma unroll
    for (int i = 0; i < RMS_MAXC; i++)
      if (i < d / 2048) xv[i] = xr[tid + 256 * i];
#pragma unroll
    for (int i = 0; i < RMS_MAXC; i++) {
      if (i < d / 2048) {
        const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float a = lo_bf(w[e]), b = hi_bf(w[e]);
          ss = fmaf(a, a, ss);
          ss = fmaf(b, b, ss);
        }
      }
    }
  } else {
    for (int c = tid; c < d; c += 256) {
      const float v = ld(x, base + c, dt);
      ss = fmaf(v, v, ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.f / sqrtf(tot / float(d) + eps);
  if (vec) {
    const u32x4* gr = reinterpret_cast<const u32x4*>(g);
    u32x4* yr = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + base);
#pragma unroll
    for (int i = 0; i < RMS_MAXC; i++) {
      if (i < d / 2048) {
        const u32x4 gv = gr[tid + 256 * i];
        const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = pack_bf2(lo_bf(w[e]) * inv * lo_bf(gw[e]), hi_bf(w[e]) * inv * hi_bf(gw[e]));
        yr[tid + 256 * i] = u32x4{o[0], o[1], o[2], o[3]};
      }
    }
  } else {
    for (int c = tid; c < d; c += 256) st(y, base + c, ld(x, base + c, dt) * inv * ld(g, c, dt), dt);
  }
}

// The residual step of a projection and the RMSNorm that follows it, one workgroup per row (bf16,
// d a multiple of 2048): h[r] += sum over the S split-K partials P[s][r] (summed in ascending s,
// then added and rounded to bf16, as the projection's residual epilogue does), then
// y[r] = rmsnorm(h[r]) * g with the reduction of rmsnorm_kernel.  Both results equal the two
// kernels' bit for bit; the new row is stored and normalised from registers.
__global__ __launch_bounds__(256) void resid_rmsnorm_kernel(const float* __restrict__ P, int S, int M, void* h,
                                                            const void* g, void* y, int d, float eps) {
  __shared__ float red[4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = int64_t(r) * d;
  const int64_t pst = int64_t(M) * d;  // between the partials of consecutive splits
  u32x4* hr = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(h) + base);
  u32x4 xv[RMS_MAXC];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < RMS_MAXC; i++) {
    if (i < d / 2048) {
      const int c0 = 8 * (tid + 256 * i);
      const f32x4* p = reinterpret_cast<const f32x4*>(P + base + c0);
      f32x4 a = p[0], b = p[1];
      // the partials of up to eight splits are loaded together, then added in ascending order
      for (int s0 = 1; s0 < S; s0 += 8) {
        f32x4 ta[8], tb[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
          if (s0 + k < S) {
            const f32x4* q = reinterpret_cast<const f32x4*>(P + (s0 + k) * pst + base + c0);
            ta[k] = q[0];
            tb[k] = q[1];
          }
        }
#pragma unroll
        for (int k = 0; k < 8; k++) {
          if (s0 + k < S) {
            a += ta[k];
            b += tb[k];
          }
        }
      }
      const u32x4 hv = hr[tid + 256 * i];
      const uint32_t w[4] = {hv.x, hv.y, hv.z, hv.w};
      const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; e++) o[e] = pack_bf2(lo_bf(w[e]) + v[2 * e], hi_bf(w[e]) + v[2 * e + 1]);
      xv[i] = u32x4{o[0], o[1], o[2], o[3]};
      hr[tid + 256 * i] = xv[i];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const float x0 = lo_bf(o[e]), x1 = hi_bf(o[e]);
        ss = fmaf(x0, x0, ss);
        ss = fmaf(x1, x1, ss);
      }
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.f / sqrtf(tot / float(d) + eps);
  const u32x4* gr = reinterpret_cast<const u32x4*>(g);
  u32x4* yr = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + base);
#pragma unroll
  for (int i = 0; i < RMS_MAXC; i++) {
    if (i < d / 2048) {
      const u32x4 gv = gr[tid + 256 * i];
      const uint32_t w[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; e++) o[e] = pack_bf2(lo_bf(w[e]) * inv * lo_bf(gw[e]), hi_bf(w[e]) * inv * hi_bf(gw[e]));
      yr[tid + 256 * i] = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

// Greedy choice per row: the largest logit, ties to the lowest index; -1 when the row has no
// finite maximum (every logit NaN, or all of them -inf), which no embedding row answers to.
__global__ __launch_bounds__(1024) void argmax_kernel(const float* logits, int V, int32_t* out) {
  __shared__ float bv[1024];
  __shared__ int bi[1024];
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* p = logits + int64_t(r) * V;
  float best = -__builtin_huge_valf();
  int bidx = 0x7fffffff;
  for (int c = tid; c < V; c += 1024) {
    const float v = p[c];
    if (v > best) {  // ascending c per thread: strict > keeps the lowest index of ties
      best = v;
      bidx = c;
    }
  }
  bv[tid] = best;
  bi[tid] = bidx;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (tid < off) {
      const float v2 = bv[tid + off];
      const int i2 = bi[tid + off];
      if (v2 > bv[tid] || (v2 == bv[tid] && i2 < bi[tid])) {
        bv[tid] = v2;
        bi[tid] = i2;
      }
    }
    __syncthreads();
  }
  if (tid == 0) out[r] = (bi[0] < V && bv[0] > -__builtin_huge_valf()) ? bi[0] : -1;
}

// a = first i < x with draft[i] != verified[i] (else x); result = [a, draft[0..a), verified[a]];
// rows[0] = verified[a] (draft = rows + 1 is read completely before rows[0] is written).
__global__ void accept_kernel(int32_t* rows, const int32_t* verified, int x, int32_t* result) {
  if (threadIdx.x != 0) return;
  const int32_t* draft = rows + 1;
  int a = x;
  for (int i = 0; i < x; i++) {
    if (draft[i] != verified[i]) {
      a = i;
      break;
    }
  }
  result[0] = a;
  for (int i = 0; i < a; i++) result[1 + i] = draft[i];
  const int32_t next = verified[a];
  result[1 + a] = next;
  rows[0] = next;
}

// tok[r] = *src[r] and, after the step, *dst[r] = out[r] (per-request token slots).
struct TokPtrs {
  const int32_t* src[VC_MAX_BATCH];
  int32_t* dst[VC_MAX_BATCH];
  int32_t n;
};
__global__ void gather_tok_kernel(const TokPtrs p, int32_t* tok) {
  const int r = threadIdx.x;
  if (r < p.n) tok[r] = *p.src[r];
}
__global__ void scatter_tok_kernel(const TokPtrs p, const int32_t* out) {
  const int r = threadIdx.x;
  if (r < p.n) *p.dst[r] = out[r];
}

// Copy rows 0..result[0] of vtail into tail at row n_tail, for every (layer, head).
__global__ void commit_rows_kernel(const uint8_t* vk, const uint8_t* vv, int vcap, uint8_t* tk, uint8_t* tv, int tcap,
                                   int n_tail, int row_bytes, int n_lh, const int32_t* result) {
  const int a = result[0];
  const int row = blockIdx.y;
  if (row > a) return;
  const int lh = blockIdx.z;
  const int words = row_bytes / 4;
  for (int w = threadIdx.x; w < words; w += blockDim.x) {
    const int64_t so = (int64_t(lh) * vcap + row) * row_bytes;
    const int64_t dof = (int64_t(lh) * tcap + n_tail + row) * row_bytes;
    reinterpret_cast<uint32_t*>(tk + dof)[w] = reinterpret_cast<const uint32_t*>(vk + so)[w];
    reinterpret_cast<uint32_t*>(tv + dof)[w] = reinterpret_cast<const uint32_t*>(vv + so)[w];
  }
}

// cos/sin of pos * theta^(-2i/D) in float64, stored float32 [max_pos][D/2][2].
__global__ void rope_table_kernel(float* tab, int max_pos, int D, double theta) {
  const int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int half = D / 2;
  if (u >= int64_t(max_pos) * half) return;
  const int i = int(u % half);
  const int64_t pos = u / half;
  const double ang = double(pos) * pow(theta, -2.0 * double(i) / double(D));
  tab[2 * u] = float(cos(ang));
  tab[2 * u + 1] = float(sin(ang));
}

__global__ void copy_words_kernel(const uint32_t* src, uint32_t* dst, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace

static inline int64_t ebytes(int dt) { return dt == VC_BF16 ? 2 : 4; }

vc_status k_embed(const void* E, const int32_t* tok, void* h, int M, int d, int V, int dt, hipStream_t s) {
  VC_DBG_LAUNCH("embed", {"embedding table", E, int64_t(V) * d * ebytes(dt)}, {"tokens", tok, int64_t(M) * 4},
                {"rows", h, int64_t(M) * d * ebytes(dt)});
  hipLaunchKernelGGL(embed_kernel, dim3(cdiv(d, 256), M), dim3(256), 0, s, E, tok, h, d, V, dt);
  VC_LAUNCH_CHECK();
  return VC_OK;
}
vc_status k_rmsnorm(const void* x, const void* g, void* y, int M, int d, float eps, int dt, hipStream_t s) {
  VC_DBG_LAUNCH("rmsnorm", {"input", x, int64_t(M) * d * ebytes(dt)}, {"gain", g, int64_t(d) * ebytes(dt)},
                {"output", y, int64_t(M) * d * ebytes(dt)});
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(M), dim3(256), 0, s, x, g, y, d, eps, dt);
  VC_LAUNCH_CHECK();
  return VC_OK;
}
bool resid_rmsnorm_ok(int d, int dt) { return dt == VC_BF16 && d % 2048 == 0 && d <= 2048 * RMS_MAXC; }
vc_status k_resid_rmsnorm(const float* P, int S, void* h, const void* g, void* y, int M, int d, float eps, int dt,
                          hipStream_t s) {
  VC_REQUIRE(resid_rmsnorm_ok(d, dt) && S >= 1, VC_ERR_UNSUPPORTED, "resid_rmsnorm: d=%d", d);
  VC_DBG_LAUNCH("resid_rmsnorm", {"partials", P, int64_t(S) * M * d * 4}, {"residual", h, int64_t(M) * d * 2},
                {"gain", g, int64_t(d) * 2}, {"output", y, int64_t(M) * d * 2});
  hipLaunchKernelGGL(resid_rmsnorm_kernel, dim3(M), dim3(256), 0, s, P, S, M, h, g, y, d, eps);
  VC_LAUNCH_CHECK();
  return VC_OK;
}
vc_status k_argmax(const float* logits, int M, int V, int32_t* out, hipStream_t s) {
  VC_DBG_LAUNCH("argmax", {"logits", logits, int64_t(M) * V * 4}, {"tokens", out, int64_t(M) * 4});
  hipLaunchKernelGGL(argmax_kernel, dim3(M), dim3(1024), 0, s, logits, V, out);
  VC_LAUNCH_CHECK();
  return VC_OK;
}
vc_status k_accept(int32_t* rows, const int32_t* verified, int x, int32_t* result, hipStream_t s) {
  VC_DBG_LAUNCH("accept", {"rows", rows, int64_t(x + 1) * 4}, {"verified", verified, int64_t(x + 1) * 4},
                {"result", result, int64_t(x + 2) * 4});
  hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(64), 0, s, rows, verified, x, result);
  VC_LAUNCH_CHECK();
  return VC_OK;
}
vc_status k_gather_tok(const int32_t* const* src, int n, int32_t* tok, hipStream_t s) {
  if (dbg_on()) {
    for (int r = 0; r < n; r++)
      if (vc_status st = dbg_check_one("gather_tok", {"request token slot", src[r], 4})) return st;
  }
  VC_DBG_LAUNCH("gather_tok", {"tokens", tok, int64_t(n) * 4});
  TokPtrs p{};
  p.n = n;
  for (int r = 0; r < n; r++) p.src[r] = src[r];
  hipLaunchKernelGGL(gather_tok_kernel, dim3(1), dim3(64), 0, s, p, tok);
  VC_LAUNCH_CHECK();
  return VC_OK;
}
vc_status k_scatter_tok(int32_t* const* dst, int n, const int32_t* out, hipStream_t s) {
  if (dbg_on()) {
    for (int r = 0; r < n; r++)
      if (vc_status st = dbg_check_one("scatter_tok", {"request token slot", dst[r], 4})) return st;
  }
  VC_DBG_LAUNCH("scatter_tok", {"tokens", out, int64_t(n) * 4});
  TokPtrs p{};
  p.n = n;
  for (int r = 0; r < n; r++) p.dst[r] = dst[r];
  hipLaunchKernelGGL(scatter_tok_kernel, dim3(1), dim3(64), 0, s, p, out);
  VC_LAUNCH_CHECK();
  return VC_OK;
}
vc_status k_commit_rows(const void* vk, const void* vv, int vcap, void* tk, void* tv, int tcap, int n_tail,
                        int row_bytes, int n_lh, int max_rows, const int32_t* result, hipStream_t s) {
  // rows 0..result[0] (at most max_rows) of every (layer, head)
  const int64_t rb = row_bytes;
  VC_DBG_LAUNCH("commit_rows", dbg_2d("verified K rows", vk, vcap * rb, max_rows * rb, n_lh),
                dbg_2d("verified V rows", vv, vcap * rb, max_rows * rb, n_lh),
                dbg_2d("tail K rows", static_cast<uint8_t*>(tk) + n_tail * rb, tcap * rb, max_rows * rb, n_lh),
                dbg_2d("tail V rows", static_cast<uint8_t*>(tv) + n_tail * rb, tcap * rb, max_rows * rb, n_lh),
                {"accept result", result, 4});
  hipLaunchKernelGGL(commit_rows_kernel, dim3(1, max_rows, n_lh), dim3(64), 0, s, static_cast<const uint8_t*>(vk),
                     static_cast<const uint8_t*>(vv), vcap, static_cast<uint8_t*>(tk), static_cast<uint8_t*>(tv), tcap,
                     n_tail, row_bytes, n_lh, result);
  VC_LAUNCH_CHECK();
  return VC_OK;
}
vc_status k_rope_table(float* tab, int max_pos, int D, double theta, hipStream_t s) {
  VC_DBG_LAUNCH("rope_table", {"table", tab, int64_t(max_pos) * D * 4});
  const int64_t n = int64_t(max_pos) * (D / 2);
  hipLaunchKernelGGL(rope_table_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, tab, max_pos, D, theta);
  VC_LAUNCH_CHECK();
  return VC_OK;
}
vc_status k_copy_words(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 4;
  if (n == 0) return VC_OK;
  VC_DBG_LAUNCH("copy_words", {"source", src, n * 4}, {"destination", dst, n * 4});
  hipLaunchKernelGGL(copy_words_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, static_cast<const uint32_t*>(src),
                     static_cast<uint32_t*>(dst), n);
  VC_LAUNCH_CHECK();
  return VC_OK;
}

}  // namespace vc
