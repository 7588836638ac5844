// Sampled decoding: draws from softmax(logits / temperature) and speculative rejection
// sampling of a verified round ("VeriCache Guide: Lossless Inference with Lossy KV Caches",
// "Mathematical Guarantee of Lossless Correctness": a draft x is kept with probability
// min(1, p_target(x) / p_draft(x)); after a rejection the replacement comes from
// max(0, p_target - p_draft) renormalised).
//
// Uniforms: Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
// 1, 2, 3", SC 2011) with key (seed, 0) and counter (position, purpose, stream, 0); the draw is
// (first output word >> 40) * 2^-24, a multiple of 2^-24 in [0, 1), exact in fp32.
//
// One workgroup of 1024 threads handles one row of V logits.  Every pass over the row is a
// fixed-order computation, so a row's result depends only on that row:
//   stats:  the largest finite logit (lowest index on ties) and whether the row holds NaN or
//           +inf (such a row, or one with nothing finite, draws -1);
//   sum:    weights w_i (exp((l_i - max) / temperature), or the residual max(0, p_t - p_d)),
//           taken in scan blocks of 4096 elements: thread t owns elements 4t..4t+3 of a block,
//           a wave scans its threads' sums with shuffles, the 16 wave totals go through LDS and
//           are added in wave order; the row total S is the blocks' totals added in order;
//   find:   the same blocks again, with the running sum C_i = (carry + before-thread) + local
//           prefix; the token is the lowest index i with w_i > 0 and C_i > u * S (if rounding
//           leaves none, the last index of positive weight);
//   probs:  optionally p_i = w_i / S for the whole row.
// Temperature 0 gives the one-hot distribution at the greedy argmax, which every rule above
// then reduces to.
#include <climits>

#include "bounds.h"
#include "sampling.h"

namespace vc {

namespace {

constexpr int ST = 1024;       // threads per row
constexpr int SWV = ST / 64;   // waves per row
constexpr int SB = 4 * ST;     // elements per scan block

// ---------------------------------------------------------------- Philox4x64-10
constexpr uint64_t PH_M0 = 0xD2E7470EE14C6C93ull, PH_M1 = 0xCA5A826395121157ull;
constexpr uint64_t PH_W0 = 0x9E3779B97F4A7C15ull, PH_W1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                                                 uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; r++) {
    if (r) {
      k0 += PH_W0;
      k1 += PH_W1;
    }
    const uint64_t lo0 = PH_M0 * c0, hi0 = __umul64hi(PH_M0, c0);
    const uint64_t lo1 = PH_M1 * c2, hi1 = __umul64hi(PH_M1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

__device__ __forceinline__ float draw(uint64_t seed, uint64_t stream, int64_t pos, int purpose) {
  const uint64_t r = philox_word0(uint64_t(pos), uint64_t(purpose), stream, 0, seed, 0);
  return float(uint32_t(r >> 40)) * 0x1p-24f;
}

// ---------------------------------------------------------------- row statistics
struct RowStat {
  float m;  // largest finite logit (-inf if none)
  int idx;  // its lowest index
  int bad;  // NaN or +inf present, or nothing finite
};

__device__ RowStat row_stat(const float* l, int V, float* redf, int* redi) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float best = NEG_INF;
  int bi = INT_MAX, bad = 0;
  for (int i = tid; i < V; i += ST) {  // ascending per thread: strict > keeps the lowest index
    const float v = l[i];
    bad |= (v != v) | (v == -NEG_INF);
    if (v > best) {
      best = v;
      bi = i;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v2 = __shfl_xor(best, o, 64);
    const int i2 = __shfl_xor(bi, o, 64);
    if (v2 > best || (v2 == best && i2 < bi)) {
      best = v2;
      bi = i2;
    }
  }
  if (lane == 0) {
    redf[wave] = best;
    redi[wave] = bi;
  }
  bad = __syncthreads_or(bad);
  RowStat r{redf[0], redi[0], bad};
  for (int w = 1; w < SWV; w++)
    if (redf[w] > r.m || (redf[w] == r.m && redi[w] < r.idx)) {
      r.m = redf[w];
      r.idx = redi[w];
    }
  __syncthreads();  // redf / redi are free again
  if (!(r.m > NEG_INF)) r.bad = 1;
  return r;
}

// ---------------------------------------------------------------- weights
// exp((l_i - m) / tau), or the one-hot row at the greedy index when tau == 0
struct TargetW {
  const float* l;
  float m, tau;
  int idx;
  __device__ __forceinline__ float operator()(int i) const {
    return tau > 0.f ? expf((l[i] - m) / tau) : (i == idx ? 1.f : 0.f);
  }
};
// max(0, p_t - p_d) with p_t = w_t / S_t
struct ResidW {
  TargetW t;
  float S;
  const float* pd;
  __device__ __forceinline__ float operator()(int i) const { return fmaxf(0.f, t(i) / S - pd[i]); }
};
// p_t without one excluded index (the fallback after a rejection whose residual has no mass)
struct ExclW {
  TargetW t;
  int ex;
  __device__ __forceinline__ float operator()(int i) const { return i == ex ? 0.f : t(i); }
};

// One scan block starting at element `base`: this thread's four weights w[], their local
// inclusive sums c[], the sum of the block's weights before this thread (ex) and the block total
// (bt).  tot: LDS [2][SWV] wave totals, double-buffered by block parity so that one barrier per
// block suffices.
template <class WF>
__device__ __forceinline__ void scan_block(const WF& wf, int V, int base, int parity, float* tot, float w[4],
                                           float c[4], float& ex, float& bt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = base + 4 * tid;
#pragma unroll
  for (int k = 0; k < 4; k++) w[k] = i0 + k < V ? wf(i0 + k) : 0.f;
  c[0] = w[0];
  c[1] = c[0] + w[1];
  c[2] = c[1] + w[2];
  c[3] = c[2] + w[3];
  float incl = c[3];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  float lex = __shfl_up(incl, 1, 64);
  if (lane == 0) lex = 0.f;
  const float wt = __shfl(incl, 63, 64);
  float* tp = tot + parity * SWV;
  if (lane == 0) tp[wave] = wt;
  __syncthreads();
  float wb = 0.f, all = 0.f;
  for (int k = 0; k < SWV; k++) {
    const float t = tp[k];
    if (k < wave) wb += t;
    all += t;
  }
  ex = wb + lex;
  bt = all;
}

// Row total of the weights, and the last index of positive weight (-1 if none).
template <class WF>
__device__ float weight_sum(const WF& wf, int V, float* tot, int* redi, int& last_pos) {
  float carry = 0.f;
  int lp = -1;
  for (int base = 0, b = 0; base < V; base += SB, b++) {
    float w[4], c[4], ex, bt;
    scan_block(wf, V, base, b & 1, tot, w, c, ex, bt);
    carry += bt;
#pragma unroll
    for (int k = 0; k < 4; k++)
      if (w[k] > 0.f) lp = base + 4 * int(threadIdx.x) + k;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lp = max(lp, __shfl_xor(lp, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) redi[threadIdx.x >> 6] = lp;
  __syncthreads();
  last_pos = -1;
  for (int k = 0; k < SWV; k++) last_pos = max(last_pos, redi[k]);
  __syncthreads();
  return carry;
}

// The lowest index i with w_i > 0 and C_i > target, or -1.
template <class WF>
__device__ int weight_find(const WF& wf, int V, float target, float* tot, int* shared_idx) {
  if (threadIdx.x == 0) *shared_idx = INT_MAX;
  __syncthreads();
  float carry = 0.f;
  for (int base = 0, b = 0; base < V; base += SB, b++) {
    float w[4], c[4], ex, bt;
    scan_block(wf, V, base, b & 1, tot, w, c, ex, bt);
    const float pre = carry + ex;
    int cand = INT_MAX;
#pragma unroll
    for (int k = 3; k >= 0; k--)
      if (w[k] > 0.f && pre + c[k] > target) cand = base + 4 * int(threadIdx.x) + k;
    if (__syncthreads_or(cand != INT_MAX)) {
      if (cand != INT_MAX) atomicMin(shared_idx, cand);
      __syncthreads();
      const int k = *shared_idx;
      __syncthreads();  // every thread has read it before the next call resets it
      return k;
    }
    carry += bt;
  }
  return -1;
}

// Draw from the weights with uniform u (their sum S and last positive index given).
template <class WF>
__device__ int weight_draw(const WF& wf, int V, float S, int last_pos, float u, float* tot, int* shared_idx) {
  const int k = weight_find(wf, V, u * S, tot, shared_idx);
  return k >= 0 ? k : last_pos;
}

struct SampleArgs {
  SampleRow r[SAMPLE_MAX_ROWS];
  int V, purpose;
};

__global__ __launch_bounds__(ST) void sample_kernel(SampleArgs a) {
  __shared__ float tot[2 * SWV];
  __shared__ float redf[SWV];
  __shared__ int redi[SWV];
  __shared__ int sidx;
  const SampleRow& R = a.r[blockIdx.x];
  const int V = a.V;
  const RowStat st = row_stat(R.logits, V, redf, redi);
  if (st.bad) {
    if (threadIdx.x == 0) *R.out = -1;
    if (R.probs)
      for (int i = threadIdx.x; i < V; i += ST) R.probs[i] = __builtin_nanf("");
    return;
  }
  const TargetW wf{R.logits, st.m, R.tau, st.idx};
  int last;
  const float S = weight_sum(wf, V, tot, redi, last);
  const float u = draw(R.seed, R.stream, R.pos, a.purpose);
  const int tok = weight_draw(wf, V, S, last, u, tot, &sidx);
  if (threadIdx.x == 0) *R.out = tok;
  if (R.probs)
    for (int i = threadIdx.x; i < V; i += ST) R.probs[i] = wf(i) / S;
}

// ---------------------------------------------------------------- speculative rejection sampling
// Per verify row (x + 1 of them): max, greedy index, bad flag, S_t and the acceptance of draft i.
struct SpecStat {
  float m, S;
  int idx, bad, acc, pad[3];
};
static_assert(sizeof(SpecStat) == 32, "spec workspace row");

__global__ __launch_bounds__(ST) void spec_rows_kernel(const float* logits_t, const float* probs_d,
                                                       const int32_t* draft, int x, int V, float tau, uint64_t seed,
                                                       uint64_t stream, int64_t pos0, SpecStat* ws) {
  __shared__ float tot[2 * SWV];
  __shared__ float redf[SWV];
  __shared__ int redi[SWV];
  const int i = blockIdx.x;
  const float* l = logits_t + int64_t(i) * V;
  const RowStat st = row_stat(l, V, redf, redi);
  SpecStat o{};
  o.m = st.m;
  o.idx = st.idx;
  o.bad = st.bad;
  o.S = 0.f;
  o.acc = 0;
  if (!st.bad) {
    const TargetW wf{l, st.m, tau, st.idx};
    int last;
    o.S = weight_sum(wf, V, tot, redi, last);
    if (i < x) {
      const int d = draft[i];
      if (d >= 0 && d < V) {
        const float pt = wf(d) / o.S;
        const float pd = probs_d[int64_t(i) * V + d];
        const float u = draw(seed, stream, pos0 + 1 + i, VC_DRAW_ACCEPT);
        o.acc = u * pd < pt;
      }
    }
  }
  if (threadIdx.x == 0) ws[i] = o;
}

// a = first rejected draft (else x); verified[0..a) = the kept drafts, verified[a] = the token
// drawn from the residual of row a (a < x) or from row x (the bonus).
__global__ __launch_bounds__(ST) void spec_pick_kernel(const float* logits_t, const float* probs_d,
                                                       const int32_t* draft, int x, int V, float tau, uint64_t seed,
                                                       uint64_t stream, int64_t pos0, const SpecStat* ws,
                                                       int32_t* verified) {
  __shared__ float tot[2 * SWV];
  __shared__ int redi[SWV];
  __shared__ int sidx;
  int a = x;
  for (int i = 0; i < x; i++)
    if (!ws[i].acc) {
      a = i;
      break;
    }
  for (int i = threadIdx.x; i < a; i += ST) verified[i] = draft[i];
  const SpecStat st = ws[a];
  int tok = -1;
  if (!st.bad) {
    const float* l = logits_t + int64_t(a) * V;
    const TargetW tw{l, st.m, tau, st.idx};
    const float u = draw(seed, stream, pos0 + 1 + a, VC_DRAW_TARGET);
    if (a == x) {
      int last;
      const float S = weight_sum(tw, V, tot, redi, last);  // equals st.S: the same blocks in the same order
      tok = weight_draw(tw, V, S, last, u, tot, &sidx);
    } else {
      const ResidW rw{tw, st.S, probs_d + int64_t(a) * V};
      int last;
      const float R = weight_sum(rw, V, tot, redi, last);
      if (R > 0.f) {
        tok = weight_draw(rw, V, R, last, u, tot, &sidx);
      } else {
        const ExclW ew{tw, draft[a]};
        const float S = weight_sum(ew, V, tot, redi, last);
        if (S > 0.f) tok = weight_draw(ew, V, S, last, u, tot, &sidx);
      }
    }
  }
  if (threadIdx.x == 0) verified[a] = tok;
}

}  // namespace

vc_status k_sample(const SampleRow* rows, int n, int V, int purpose, hipStream_t s) {
  VC_REQUIRE(n >= 0 && n <= SAMPLE_MAX_ROWS && V > 0, VC_ERR_ARG, "sample: %d rows of %d logits", n, V);
  if (n == 0) return VC_OK;
  if (dbg_on()) {
    for (int r = 0; r < n; r++) {
      if (vc_status st = dbg_check("sample", {{"logits", rows[r].logits, int64_t(V) * 4},
                                              {"token", rows[r].out, 4},
                                              {"probabilities", rows[r].probs, rows[r].probs ? int64_t(V) * 4 : 0}}))
        return st;
    }
    if (dbg_dry()) return VC_OK;
  }
  SampleArgs a{};
  for (int r = 0; r < n; r++) a.r[r] = rows[r];
  a.V = V;
  a.purpose = purpose;
  hipLaunchKernelGGL(sample_kernel, dim3(n), dim3(ST), 0, s, a);
  VC_LAUNCH_CHECK();
  return VC_OK;
}

size_t spec_ws_bytes(int x) { return sizeof(SpecStat) * size_t(x + 1); }

vc_status k_spec(const float* logits_t, const float* probs_d, const int32_t* draft, int x, int V, float tau,
                 uint64_t seed, uint64_t stream, int64_t pos0, int32_t* verified, void* ws, hipStream_t s) {
  VC_REQUIRE(x >= 0 && V > 0, VC_ERR_ARG, "spec: x %d, V %d", x, V);
  SpecStat* w = static_cast<SpecStat*>(ws);
  VC_DBG_LAUNCH("spec_rows", {"target logits", logits_t, int64_t(x + 1) * V * 4},
                {"draft probabilities", probs_d, int64_t(x) * V * 4}, {"drafts", draft, int64_t(x) * 4},
                {"workspace", ws, int64_t(spec_ws_bytes(x))}, {"verified", verified, int64_t(x + 1) * 4});
  hipLaunchKernelGGL(spec_rows_kernel, dim3(x + 1), dim3(ST), 0, s, logits_t, probs_d, draft, x, V, tau, seed, stream,
                     pos0, w);
  VC_LAUNCH_CHECK();
  hipLaunchKernelGGL(spec_pick_kernel, dim3(1), dim3(ST), 0, s, logits_t, probs_d, draft, x, V, tau, seed, stream,
                     pos0, w, verified);
  VC_LAUNCH_CHECK();
  return VC_OK;
}

}  // namespace vc
