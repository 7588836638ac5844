// Projection GEMMs (Y = X W^T) and the fused per-layer epilogue.
//
// Decode / verify (M <= 64) are weight-streaming: every weight is read once
// per forward.  gemm_skinny_bf16: a workgroup owns 64 output columns (16 per
// wave) and one K range; the activations are staged in a double-buffered LDS
// tile 256 columns at a time and every wave runs 16x16x32 bf16 MFMAs over all
// M rows (padded to 16) while its next two chunks of weight fragments are in flight.
// Prefill chunks (M > 64) are plain bf16 GEMMs with float32 output: gemm_tile256_bf16 (256 x 256
// tiles, eight waves of 128 x 64, two per SIMD) where N is a multiple of 256, else
// gemm_big_bf16 (128 x 128 x 32 tiles).  The fp32 model uses a 16x16 tiled VALU kernel whose
// outputs are single fma chains in ascending k.
#include <algorithm>

#include "bounds.h"
#include "gemm.h"

namespace vc {

namespace {

constexpr int SK_NB = 64;
constexpr int SK_KC = 256;
#ifndef SK_NT
#define SK_NT 1  // weight loads marked non-temporal: streamed once, they leave X and the partials in L2
#endif

// PACKED: W in the fragment-major layout of pack_weights (each wave's 16 B per lane weight loads
// read one contiguous 1 KB tile); otherwise row-major [N][K].  NMT: 16-row tiles of X (M <= 16
// NMT).  Same MFMAs in the same order for every variant.
//
// k advances SK_KC = 256 at a time.  Weights go to registers, two chunks ahead: chunk i + 2 is
// loaded into the register set chunk i has just used (two sets, alternating), so every wave has
// up to 16 KB of weights in flight.  X (M rows padded to 16 NMT) goes to a double-buffered LDS
// tile of 512-byte rows by direct-to-LDS buffer loads, one chunk ahead; the buffer resource ends
// at row M, so the padding rows load as zero.  Within a row the 16-byte chunks are XOR-swizzled
// by the row's low four bits, so the sixteen rows one fragment read touches fall in distinct
// banks.  One barrier per chunk, after a wait for this wave's loads of the chunk (X chunk i and,
// older, weight chunk i; only weight chunk i + 1 may stay in flight); it carries no memory fence,
// which would wait for every load in flight.  After it no wave still reads the other X buffer,
// which is then refilled with chunk i + 1.  Every chunk loads all eight weight tiles per lane
// (the second half of a 128-long last chunk re-reads the first half's tiles, unused), and the
// main loop (pairs of chunks, both register sets) issues its loads unconditionally, so the
// compiler's own waits before each MFMA count exactly the loads issued after its operand's.
template <bool PACKED, int NMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void gemm_skinny_bf16(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, float* __restrict__ P, int M, int N, int K,
    int kps) {
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int ROWS = 16 * NMT, NX = ROWS / 8;  // X rows in LDS; X instructions per wave and chunk
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2 * ROWS * SK_KC];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int n0 = blockIdx.x * SK_NB + wave * 16;
  const int s = blockIdx.y;
  const int k_lo = s * kps, k_hi = min(K, k_lo + kps);
  const int nch = (k_hi - k_lo + SK_KC - 1) / SK_KC;
  f32x4 acc[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; mt++) acc[mt] = f32x4{0, 0, 0, 0};
  // this wave's weights through a buffer resource: the chunk's byte offset is uniform (soffset),
  // the lane's and the tile's are the constant voffset and immediate, so a load holds no address
  // registers.  PACKED: the wave's 16 rows are K / 32 consecutive 1 KB tiles; else 16 rows of K.
  const uint16_t* wbase = PACKED ? W + int64_t(n0 >> 4) * (K >> 5) * 512 : W + int64_t(n0) * K;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wbase), 0, 16 * K * 2, BUF_DWORD3);
  const int wlane = PACKED ? 16 * lane : r * K * 2 + 16 * g;
  auto load_w = [&](u32x4(&S)[8], int i) {
    const int kc = k_lo + SK_KC * i, klen = min(SK_KC, k_hi - kc);
    const int half = 128 < klen ? 1 : 0;  // a 128-long chunk re-reads its first half as the second
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int kt = PACKED ? (kc >> 5) * 1024 : 2 * kc;                  // chunk (uniform)
        const int ko = PACKED ? (4 * h * half + e) * 1024 : 2 * (128 * h * half + 32 * e);
        S[4 * h + e] = __builtin_amdgcn_raw_buffer_load_b128(rw, wlane + (h ? 0 : ko), kt + (h ? ko : 0),
                                                             SK_NT ? 2 : 0);
      }
    }
  };
  // X chunk i -> buffer buf = i & 1 (a literal at every call): wave instruction j (= 4 t + wave) fills rows 2 j, 2 j + 1; lane ->
  // row 2 j + lane / 32, LDS slot lane % 32, which holds source chunk slot ^ (row & 15)
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), 0, M * K * 2, BUF_DWORD3);
  auto load_x = [&](int i, int buf) {
    const int kc = k_lo + SK_KC * i;
#pragma unroll
    for (int t = 0; t < NX; t++) {
      const int j = 4 * t + wave, row = 2 * j + (lane >> 5);
      const int c = (lane & 31) ^ (row & 15);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)&Xs[(buf * ROWS + 2 * j) * SK_KC], 16,
                                               row * K * 2 + 2 * (kc + 8 * c), 0, 0, 0);
    }
  };
  auto compute = [&](const u32x4(&S)[8], int i, int buf) {
    const int klen = min(SK_KC, k_hi - k_lo - SK_KC * i);
    const uint16_t* xb = Xs + (buf * ROWS + r) * SK_KC;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      if (128 * h >= klen) break;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int c = (16 * h + 4 * e + g) ^ r;
#pragma unroll
        for (int mt = 0; mt < NMT; mt++) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(xb + 16 * mt * SK_KC + 8 * c);
          acc[mt] = mfma_bf16(a, S[4 * h + e], acc[mt]);
        }
        // one k step's fragments live at a time (the chunk's MFMAs take a few hundred cycles,
        // its loads microseconds: no need to read ahead)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto sync = [&]() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  u32x4 wa[8], wb[8];
  // chunk 1 clamped to chunk 0 when there is only one: a redundant load, so the count is fixed
  load_w(wa, 0);
  load_x(0, 0);
  load_w(wb, min(1, nch - 1));
  int i = 0;
  for (; i + 3 < nch; i += 2) {  // both steps load: X chunks i + 1, i + 2, weight chunks i + 2, i + 3
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    sync();
    load_x(i + 1, 1);
    compute(wa, i, 0);
    load_w(wa, i + 2);
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    sync();
    load_x(i + 2, 0);
    compute(wb, i + 1, 1);
    load_w(wb, i + 3);
  }
  // the last one to three chunks: loads only of chunks that exist, and the wait for chunk i
  // leaves weight chunk i + 1 in flight only where it was loaded
  auto tail = [&](u32x4(&S)[8], int c, int buf) {  // X chunk c is in buffer c & 1 = buf
    if (c + 1 < nch) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    sync();
    if (c + 1 < nch) load_x(c + 1, buf ^ 1);
    compute(S, c, buf);
    if (c + 2 < nch) load_w(S, c + 2);
  };
  if (i < nch) tail(wa, i, 0);  // i is even
  if (i + 1 < nch) tail(wb, i + 1, 1);
  if (i + 2 < nch) tail(wa, i + 2, 0);
#pragma unroll
  for (int mt = 0; mt < NMT; mt++) {
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const int m = 16 * mt + 4 * g + jj;
      if (m < M) P[(int64_t(s) * M + m) * N + n0 + r] = acc[mt][jj];
    }
  }
}

template <bool PACKED>
void launch_skinny(const uint16_t* X, const uint16_t* W, float* P, int M, int N, int K, int S, int kps,
                   hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid(N / SK_NB, S);
  switch ((M + 15) / 16) {
    case 1: hipExtLaunchKernelGGL(HIP_KERNEL_NAME(gemm_skinny_bf16<PACKED, 1>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, X, W, P, M, N, K, kps); break;
    case 2: hipExtLaunchKernelGGL(HIP_KERNEL_NAME(gemm_skinny_bf16<PACKED, 2>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, X, W, P, M, N, K, kps); break;
    case 3: hipExtLaunchKernelGGL(HIP_KERNEL_NAME(gemm_skinny_bf16<PACKED, 3>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, X, W, P, M, N, K, kps); break;
    default: hipExtLaunchKernelGGL(HIP_KERNEL_NAME(gemm_skinny_bf16<PACKED, 4>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, X, W, P, M, N, K, kps); break;
  }
}

// Fragment-major copy of a row-major bf16 matrix [N][K] (N % 16 == 0, K % 32 == 0): the 16 x 32
// block (16-row block nb, 32-column block kb) is 1 KB at element (nb (K / 32) + kb) 512, in the
// order the skinny kernel's lanes read it: lane l = r + 16 g holds row 16 nb + r, columns
// 32 kb + 8 g .. + 8.  Thread = one 16-byte chunk of the output.
__global__ void pack_weights_kernel(const uint16_t* __restrict__ W, uint16_t* __restrict__ Wp, int64_t n_chunks,
                                    int K) {
  const int64_t o = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (o >= n_chunks) return;
  const int64_t kbs = K >> 5;
  const int lane = int(o & 63);
  const int64_t t = o >> 6;  // tile index nb * kbs + kb
  const int64_t nb = t / kbs, kb = t - nb * kbs;
  const int r = lane & 15, g = lane >> 4;
  *reinterpret_cast<u32x4*>(Wp + 8 * o) =
      *reinterpret_cast<const u32x4*>(W + (16 * nb + r) * int64_t(K) + 32 * kb + 8 * g);
}

constexpr int BG_P = 40;  // LDS pitch (bf16) of a 32-wide k slice

__global__ __launch_bounds__(256) void gemm_big_bf16(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                     float* __restrict__ P, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][128 * BG_P];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][128 * BG_P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * 128, n0 = blockIdx.x * 128;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int jx = 0; jx < 4; jx++) acc[i][jx] = f32x4{0, 0, 0, 0};
  u32x4 ra[2], rb[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int c = tid + 256 * i;
      const int row = c >> 2, c8 = c & 3;
      const int m = m0 + row;
      ra[i] = m < M ? *reinterpret_cast<const u32x4*>(X + int64_t(m) * K + k0 + 8 * c8) : u32x4{0, 0, 0, 0};
      rb[i] = *reinterpret_cast<const u32x4*>(W + int64_t(n0 + row) * K + k0 + 8 * c8);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int c = tid + 256 * i;
      const int row = c >> 2, c8 = c & 3;
      *reinterpret_cast<u32x4*>(&As[buf][row * BG_P + 8 * c8]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][row * BG_P + 8 * c8]) = rb[i];
    }
  };
  gload(0);
  sstore(0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < K; k0 += 32) {
    const bool more = k0 + 32 < K;
    if (more) gload(k0 + 32);
    u32x4 af[4], bfr[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      af[i] = *reinterpret_cast<const u32x4*>(&As[buf][(64 * wm + 16 * i + r) * BG_P + 8 * g]);
      bfr[i] = *reinterpret_cast<const u32x4*>(&Bs[buf][(64 * wn + 16 * i + r) * BG_P + 8 * g]);
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int jx = 0; jx < 4; jx++) acc[i][jx] = mfma_bf16(af[i], bfr[jx], acc[i][jx]);
    if (more) sstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const int m = m0 + 64 * wm + 16 * i + 4 * g + jj;
      if (m >= M) continue;
#pragma unroll
      for (int jx = 0; jx < 4; jx++) P[int64_t(m) * N + n0 + 64 * wn + 16 * jx + r] = acc[i][jx][jj];
    }
  }
}

// Prefill tile: a 256 x 256 block of P from NW waves in 2 x NW/2, each wave 128 x 512/NW (32x32x16
// MFMA tiles; NW = 8: 128 x 64, 128 float accumulators per lane, two waves per SIMD, so one
// wave's MFMAs run while the other waits at a barrier or for LDS; NW = 4: 128 x 128, one wave
// per SIMD, measured 5% slower).  k advances KS at a
// time through a ring of NST LDS stages, each A [256][KS] and B [256][KS] bf16 (NST KS 1 KB in
// all), filled by direct-to-LDS buffer loads (each wave instruction writes 1 KB of whole rows),
// so the staging holds no registers; loads run NST - 1 stages ahead of the multiplies.  Per
// stage one barrier, preceded by a wait for this wave's loads of the stage (the barrier then
// publishes every wave's); the barrier carries no memory fence, which would wait for all loads
// in flight.  In each LDS row the 16-byte chunks are XOR-swizzled by the row (each lane loads
// the global chunk that belongs at its LDS slot) so that the rows one fragment read touches
// fall in distinct banks.  X is read through a buffer resource that ends at row M, so rows of
// the last tile past M load as zero and are never stored.
constexpr int PT = 256;
#ifndef GEMM_KS
#define GEMM_KS 64  // k per LDS stage
#define GEMM_NST 2  // stages in the ring
#define GEMM_NW 8   // waves per workgroup: 4 (128 x 128 each, one per SIMD) or 8 (128 x 64, two per SIMD)
#endif

template <int KS>
__device__ __forceinline__ int pt_swz(int row) {
  if constexpr (KS == 64) return (row & 7) ^ ((row >> 3) & 1);
  else return (row >> 2) & 3;
}

template <int KS, int NST, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void gemm_tile256_bf16(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, float* __restrict__ P, int M, int N, int K) {
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int CPR = KS / 8;       // 16-byte chunks per LDS row
  constexpr int RPI = 64 / CPR;     // rows one wave instruction fills
  constexpr int NI = PT / RPI / NW; // instructions per wave, operand and stage
  constexpr int WN = NW / 2;        // waves along N (two along M)
  constexpr int JN = PT / WN / 32;  // 32-column MFMA blocks per wave
  constexpr int TOT = 4 * JN;       // MFMAs per wave and 16-deep step
  __shared__ __attribute__((aligned(16))) uint16_t lds[NST][2][PT * KS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int MT = (M + PT - 1) / PT, NT = N / PT;
  // XCD x (blocks x, x + 8, ...) takes an eighth of the tile grid, split along the longer side
  // when that side divides by eight; inside it, bands of up to 8 row tiles, rows fastest, so
  // the ~32 tiles resident on one XCD form a compact block that shares its A and B slabs.
  int u = blockIdx.x, mt0 = 0, mt = MT, nt0 = 0, nt = NT;
  if (MT % 8 == 0 && MT >= NT) {
    mt = MT / 8; mt0 = (u & 7) * mt; u >>= 3;
  } else if (NT % 8 == 0) {
    nt = NT / 8; nt0 = (u & 7) * nt; u >>= 3;
  }
  const int g = min(mt, 8), band = u / (g * nt), bs = min(g, mt - band * g), rr = u - band * g * nt;
  const int m0 = (mt0 + band * g + rr % bs) * PT, n0 = (nt0 + rr / bs) * PT;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + int64_t(m0) * K), 0, min(M - m0, PT) * K * 2, BUF_DWORD3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W + int64_t(n0) * K), 0, PT * K * 2, BUF_DWORD3);
  // wave instruction i fills tile rows RPI (NW i + wave) .. + RPI; lane: row + lane / CPR, LDS chunk lane % CPR
  const int lrow = RPI * wave + lane / CPR;
  const int voff = lrow * K * 2 + 16 * ((lane % CPR) ^ pt_swz<KS>(lrow));
  const int rstep = NW * RPI * K * 2;
  auto issue = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < NI; i++) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)&lds[buf][0][RPI * (NW * i + wave) * KS], 16,
                                               voff + i * rstep + 2 * k0, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)&lds[buf][1][RPI * (NW * i + wave) * KS], 16,
                                               voff + i * rstep + 2 * k0, 0, 0, 0);
    }
  };
  f32x16 acc[4][JN];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < JN; j++) acc[i][j] = f32x16{};
  const int nk = K / KS;
  const int lr32 = lane & 31, lh = lane >> 5;
  u32x4 af[2][4], bf[2][JN];
  auto frags = [&](int buf, int s, int slot) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int ra_ = 128 * wm + 32 * i + lr32;
      af[slot][i] = *reinterpret_cast<const u32x4*>(&lds[buf][0][ra_ * KS + 8 * ((2 * s + lh) ^ pt_swz<KS>(ra_))]);
    }
#pragma unroll
    for (int j = 0; j < JN; j++) {
      const int rb_ = 32 * JN * wn + 32 * j + lr32;
      bf[slot][j] = *reinterpret_cast<const u32x4*>(&lds[buf][1][rb_ * KS + 8 * ((2 * s + lh) ^ pt_swz<KS>(rb_))]);
    }
  };
  // MFMAs number e0 .. e1 - 1 of a step (e = JN i + j: A block i, B block j)
  auto mfmas = [&](int slot, int e0, int e1) {
#pragma unroll
    for (int e = e0; e < e1; e++) acc[e / JN][e % JN] = mfma32_bf16(af[slot][e / JN], bf[slot][e % JN], acc[e / JN][e % JN]);
  };
  auto issue_one = [&](int k0, int buf, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)&lds[buf][0][RPI * (NW * i + wave) * KS], 16,
                                             voff + i * rstep + 2 * k0, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)&lds[buf][1][RPI * (NW * i + wave) * KS], 16,
                                             voff + i * rstep + 2 * k0, 0, 0, 0);
  };
  constexpr int S = KS / 16;  // 32x32x16 steps per stage
  static_assert(S % 2 == 0, "a stage's first step must use fragment slot 0");
  // The ring holds NST stages.  At the barrier of stage kt every wave has its fragments of
  // stage kt in registers (LDS reads waited for), so the buffer of stage kt is free and is
  // refilled with stage kt + NST, its loads interleaved with the stage's last MFMAs.  Each
  // step issues two MFMAs, then the LDS reads of the next step (the next stage's first step
  // after the barrier), then its other fourteen MFMAs, so every fragment is read fourteen
  // MFMAs before its first use; scheduling fences keep the compiler from pulling uses closer.
  // Stages past the last reload the last one: every load is unconditional and in range, and
  // each wave always has the same number in flight.
#pragma unroll
  for (int st = 0; st < NST; st++) issue(KS * min(st, nk - 1), st);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NI * (NST - 1)) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  frags(0, 0, 0);
  for (int kt = 0; kt < nk; kt++) {
    const int buf = kt % NST;
#pragma unroll
    for (int s = 0; s + 1 < S; s++) {
      mfmas(s & 1, 0, 2);
      __builtin_amdgcn_sched_barrier(0);
      frags(buf, s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s & 1, 2, TOT);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * NI * (NST - 2)) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    constexpr int L = (S - 1) & 1;
    mfmas(L, 0, 2);
    __builtin_amdgcn_sched_barrier(0);
    frags((kt + 1) % NST, 0, S & 1);
    __builtin_amdgcn_sched_barrier(0);
    const int kn = KS * min(kt + NST, nk - 1);
    // the step's other MFMAs with the NI load pairs spread over them
#pragma unroll
    for (int q = 0; q < NI; q++) {
      issue_one(kn, buf, q);
      mfmas(L, 2 + (TOT - 2) * q / NI, 2 + (TOT - 2) * (q + 1) / NI);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // no load may still be writing this workgroup's LDS when it ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // D element e of lane l: row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int e = 0; e < 16; e++) {
      const int m = m0 + 128 * wm + 32 * i + 8 * (e >> 2) + 4 * lh + (e & 3);
      if (m >= M) continue;
      float* prow = P + int64_t(m) * N + n0 + 32 * JN * wn + lr32;
#pragma unroll
      for (int j = 0; j < JN; j++) prow[32 * j] = acc[i][j][e];
    }
  }
}

__global__ __launch_bounds__(256) void gemm_f32_tiled(const float* __restrict__ X, const float* __restrict__ W,
                                                      float* __restrict__ P, int M, int N, int K) {
  __shared__ float Xs[16][17];
  __shared__ float Ws[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m = blockIdx.y * 16 + ty, n = blockIdx.x * 16 + tx;
  float acc = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
    const int xm = blockIdx.y * 16 + ty, wn = blockIdx.x * 16 + ty;
    Xs[ty][tx] = (xm < M && k0 + tx < K) ? X[int64_t(xm) * K + k0 + tx] : 0.f;
    Ws[ty][tx] = (wn < N && k0 + tx < K) ? W[int64_t(wn) * K + k0 + tx] : 0.f;
    __syncthreads();
    const int kl = min(16, K - k0);
    for (int kk = 0; kk < kl; kk++) acc = fmaf(Xs[ty][kk], Ws[tx][kk], acc);
    __syncthreads();
  }
  if (m < M && n < N) P[int64_t(m) * N + n] = acc;
}

// ---------------------------------------------------------------- epilogue
__device__ __forceinline__ float ld_act(const void* p, int64_t i, int dtype) {
  return dtype == VC_BF16 ? bf2f(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}
__device__ __forceinline__ void st_act(void* p, int64_t i, float v, int dtype) {
  if (dtype == VC_BF16) static_cast<uint16_t*>(p)[i] = f2bf(v);
  else static_cast<float*>(p)[i] = v;
}
__device__ __forceinline__ float psum(const float* P, int S, int M, int N, int r, int c) {
  float v = P[int64_t(r) * N + c];
  for (int s = 1; s < S; s++) v += P[(int64_t(s) * M + r) * N + c];
  return v;
}

__global__ void epilogue_kernel(const EpiArgs a) {
  const int r = blockIdx.y;
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  const int M = a.M, N = a.N, S = a.S;
  if (a.mode == EPI_RESID) {
    if (u >= N) return;
    const float y = psum(a.P, S, M, N, r, u);
    const int64_t i = int64_t(r) * N + u;
    st_act(a.out, i, ld_act(a.out, i, a.dtype) + y, a.dtype);
  } else if (a.mode == EPI_SWIGLU) {
    const int F = N / 2;
    if (u >= F) return;
    const float gt = psum(a.P, S, M, N, r, u);
    const float up = psum(a.P, S, M, N, r, F + u);
    const float sg = gt / (1.f + expf(-gt));
    st_act(a.out, int64_t(r) * F + u, sg * up, a.dtype);
  } else if (a.mode == EPI_COPY) {
    if (u >= N) return;
    static_cast<float*>(a.out)[int64_t(r) * N + u] = psum(a.P, S, M, N, r, u);
  } else {  // EPI_QKV: units = (Hq + 2 Hkv) * D / 2
    const int D = a.D, half = D / 2;
    const int nq = a.Hq * half, nk = a.Hkv * half;
    if (u >= nq + 2 * nk) return;
    const int pos = a.batched ? a.pos[r] : a.pos0 + r;
    if (u < nq + nk) {
      const bool isq = u < nq;
      const int uu = isq ? u : u - nq;
      const int h = uu / half, i = uu % half;
      const int col = (isq ? 0 : a.Hq * D) + h * D + i;
      const float ya = psum(a.P, S, M, N, r, col);
      const float yb = psum(a.P, S, M, N, r, col + half);
      const float c = a.rope[(int64_t(pos) * half + i) * 2];
      const float sn = a.rope[(int64_t(pos) * half + i) * 2 + 1];
      const float oa = ya * c - yb * sn;
      const float ob = yb * c + ya * sn;
      if (isq) {
        const int64_t qi = (int64_t(r) * a.Hq + h) * D + i;
        st_act(a.q_out, qi, oa, a.dtype);
        st_act(a.q_out, qi + half, ob, a.dtype);
      } else {
        void* base;
        int64_t off;
        if (a.batched) {
          base = a.krow[r];
          off = int64_t(h) * a.rpitch[r] * D + i;
        } else {
          base = a.kbase;
          off = (int64_t(h) * a.pitch + a.row0 + r) * D + i;
        }
        st_act(base, off, oa, a.dtype);
        st_act(base, off + half, ob, a.dtype);
      }
    } else {
      const int uu = u - nq - nk;  // v pair
      const int h = uu / half, i = uu % half;
      const int col = (a.Hq + a.Hkv) * D + h * D + 2 * i;
      const float y0 = psum(a.P, S, M, N, r, col);
      const float y1 = psum(a.P, S, M, N, r, col + 1);
      void* base;
      int64_t off;
      if (a.batched) {
        base = a.vrow[r];
        off = int64_t(h) * a.rpitch[r] * D + 2 * i;
      } else {
        base = a.vbase;
        off = (int64_t(h) * a.pitch + a.row0 + r) * D + 2 * i;
      }
      st_act(base, off, y0, a.dtype);
      st_act(base, off + 1, y1, a.dtype);
    }
  }
}

}  // namespace

int gemm_splits(int M, int N, int K, int dtype) {
  if (dtype != VC_BF16 || M > 64) return 1;
  const int col_blocks = N / SK_NB;
  int want = std::max(1, 1024 / std::max(col_blocks, 1));
  const int max_s = std::max(1, K / 128);
  want = std::min(want, max_s);
  // K range per split: multiple of 128
  const int kps = int(cdiv(cdiv(K, want), 128) * 128);
  return int(cdiv(K, kps));
}

vc_status pack_weights(const void* W, void* Wp, int64_t N, int K, hipStream_t s) {
  VC_REQUIRE(N % 16 == 0 && K % 32 == 0, VC_ERR_ARG, "pack_weights: %lld x %d not 16 x 32 blocks", (long long)N, K);
  const int64_t n_chunks = N * K / 8;
  VC_DBG_LAUNCH("pack_weights", {"weights", W, N * K * 2}, {"packed weights", Wp, N * K * 2});
  hipLaunchKernelGGL(pack_weights_kernel, dim3(unsigned(cdiv(n_chunks, 256))), dim3(256), 0, s,
                     static_cast<const uint16_t*>(W), static_cast<uint16_t*>(Wp), n_chunks, K);
  VC_LAUNCH_CHECK();
  return VC_OK;
}

vc_status gemm(const void* X, const void* W, float* P, int M, int N, int K, int S, int dtype, hipStream_t s,
               hipEvent_t ev_start, hipEvent_t ev_stop, const void* Wp) {
  VC_REQUIRE(M > 0 && N > 0 && K > 0, VC_ERR_ARG, "gemm: bad shape %d x %d x %d", M, N, K);
  const bool packed = Wp != nullptr && dtype == VC_BF16 && M <= 64;
  {
    const int64_t eb = dtype == VC_BF16 ? 2 : 4;
    const int64_t parts = (dtype == VC_BF16 && M <= 64) ? S : 1;  // split-K partials of the skinny kernel
    VC_DBG_LAUNCH("gemm", {"activations", X, int64_t(M) * K * eb}, {"weights", packed ? Wp : W, int64_t(N) * K * eb},
                  {"partials", P, parts * M * N * 4});
  }
  if (dtype == VC_BF16) {
    VC_REQUIRE(K % 128 == 0, VC_ERR_UNSUPPORTED, "gemm: K=%d not a multiple of 128", K);
    if (M <= 64) {
      VC_REQUIRE(N % SK_NB == 0, VC_ERR_UNSUPPORTED, "gemm: N=%d not a multiple of 64", N);
      const int want = S;
      const int kps = int(cdiv(cdiv(K, want), 128) * 128);
      VC_REQUIRE(cdiv(K, kps) == S, VC_ERR_ARG, "gemm: split count %d inconsistent", S);
      VC_REQUIRE(K <= (1 << 20), VC_ERR_UNSUPPORTED, "gemm: K=%d beyond the 32-bit X offsets", K);
      if (packed)
        launch_skinny<true>(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(Wp), P, M, N, K, S, kps, s,
                            ev_start, ev_stop);
      else
        launch_skinny<false>(static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(W), P, M, N, K, S, kps, s,
                             ev_start, ev_stop);
    } else {
      VC_REQUIRE(S == 1, VC_ERR_ARG, "gemm: prefill tiles use one split");
      if (N % PT == 0 && K <= (1 << 20)) {  // tile offsets (256 K 2 bytes) stay within 32 bits
        const int T = int(cdiv(M, PT)) * (N / PT);
        hipExtLaunchKernelGGL(HIP_KERNEL_NAME(gemm_tile256_bf16<GEMM_KS, GEMM_NST, GEMM_NW>), dim3(T), dim3(64 * GEMM_NW), 0, s, ev_start, ev_stop, 0,
                              static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(W), P, M, N, K);
      } else {
        VC_REQUIRE(N % 128 == 0, VC_ERR_UNSUPPORTED, "gemm: N=%d not a multiple of 128", N);
        hipExtLaunchKernelGGL(gemm_big_bf16, dim3(N / 128, cdiv(M, 128)), dim3(256), 0, s, ev_start, ev_stop, 0,
                              static_cast<const uint16_t*>(X), static_cast<const uint16_t*>(W), P, M, N, K);
      }
    }
  } else {
    VC_REQUIRE(S == 1, VC_ERR_ARG, "gemm: fp32 path uses one split");
    hipExtLaunchKernelGGL(gemm_f32_tiled, dim3(cdiv(N, 16), cdiv(M, 16)), dim3(256), 0, s, ev_start, ev_stop, 0,
                          static_cast<const float*>(X), static_cast<const float*>(W), P, M, N, K);
  }
  VC_LAUNCH_CHECK();
  return VC_OK;
}

vc_status epilogue(const EpiArgs& a, hipStream_t s) {
  int units;
  switch (a.mode) {
    case EPI_QKV: units = (a.Hq + 2 * a.Hkv) * a.D / 2; break;
    case EPI_SWIGLU: units = a.N / 2; break;
    default: units = a.N; break;
  }
  VC_REQUIRE(!a.batched || a.M <= EPI_MAX_ROWS, VC_ERR_ARG, "epilogue: too many batched rows");
  if (dbg_on()) {
    const int64_t eb = a.dtype == VC_BF16 ? 2 : 4;
    const int64_t M = a.M, N = a.N;
    if (vc_status st = dbg_check_one("epilogue", {"partials", a.P, int64_t(a.S) * M * N * 4})) return st;
    vc_status st = VC_OK;
    if (a.mode == EPI_RESID) st = dbg_check("epilogue", {{"residual", a.out, M * N * eb}});
    else if (a.mode == EPI_SWIGLU) st = dbg_check("epilogue", {{"ffn activations", a.out, M * (N / 2) * eb}});
    else if (a.mode == EPI_COPY) st = dbg_check("epilogue", {{"output", a.out, M * N * 4}});
    else {
      const int64_t D = a.D, row = D * eb;
      int max_pos = a.pos0 + a.M - 1;
      if (a.batched)
        for (int r = 0; r < a.M; r++) max_pos = r ? std::max(max_pos, a.pos[r]) : a.pos[r];
      st = dbg_check("epilogue", {{"queries", a.q_out, M * a.Hq * row}, {"RoPE table", a.rope, (max_pos + 1) * D * 4}});
      for (int r = 0; r < a.M && !st && a.batched; r++) {
        st = dbg_check_one("epilogue", dbg_2d("new K row", a.krow[r], int64_t(a.rpitch[r]) * row, row, a.Hkv));
        if (!st) st = dbg_check_one("epilogue", dbg_2d("new V row", a.vrow[r], int64_t(a.rpitch[r]) * row, row, a.Hkv));
      }
      if (!st && !a.batched) {
        st = dbg_check_one("epilogue", dbg_2d("new K rows", static_cast<uint8_t*>(a.kbase) + a.row0 * row,
                                              int64_t(a.pitch) * row, M * row, a.Hkv));
        if (!st)
          st = dbg_check_one("epilogue", dbg_2d("new V rows", static_cast<uint8_t*>(a.vbase) + a.row0 * row,
                                                int64_t(a.pitch) * row, M * row, a.Hkv));
      }
    }
    if (st) return st;
    if (dbg_dry()) return VC_OK;
  }
  hipLaunchKernelGGL(epilogue_kernel, dim3(cdiv(units, 256), a.M), dim3(256), 0, s, a);
  VC_LAUNCH_CHECK();
  return VC_OK;
}

}  // namespace vc
