// Internal interface of the projection GEMMs and their fused epilogue.
//
// Y = X W^T with X [M][K] and W [N][K] (row-major, model dtype).  Every GEMM
// writes float32 partials P[s][M][N] over S disjoint K ranges; the epilogue
// sums them in ascending s and applies the layer's pointwise step.  S and the
// K order inside each range depend only on (N, K), never on M, so every output
// row's arithmetic is independent of how many rows share the call.
#pragma once
#include "common.h"

namespace vc {

int gemm_splits(int M, int N, int K, int dtype);
// Partials for M <= 64 (decode / verify): weight-streaming bf16 MFMA kernel or fp32 VALU kernel.
// Larger M (prefill chunks) uses the tiled bf16 MFMA kernel with S = 1.
// ev_start / ev_stop (optional) are recorded at the kernel's own start and end.
// Wp (optional): W in the fragment-major layout of pack_weights, used by the skinny bf16 kernel.
vc_status gemm(const void* X, const void* W, float* P, int M, int N, int K, int S, int dtype, hipStream_t s,
               hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr, const void* Wp = nullptr);
// Fragment-major copy of the bf16 matrix (or stack of matrices) W [N][K] into Wp (same size):
// 1 KB tiles of 16 rows x 32 columns, each in the lane order of the skinny kernel's loads.
vc_status pack_weights(const void* W, void* Wp, int64_t N, int K, hipStream_t s);

enum EpiMode { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_COPY = 3 };

constexpr int EPI_MAX_ROWS = VC_MAX_BATCH;

struct EpiArgs {
  const float* P;
  int32_t M, N, S, mode, dtype;
  // EPI_RESID: h[M][N] += sum;  EPI_SWIGLU: out[M][N/2];  EPI_COPY: out float [M][N]
  void* out;
  // EPI_QKV
  void* q_out;                 // [M][Hq][D]
  const float* rope;           // [max_pos][D/2][2]
  int32_t Hq, Hkv, D;
  int32_t batched;             // 1: per-row pos/k/v below (M <= EPI_MAX_ROWS); 0: strided
  int32_t pos0;                // strided: row r at position pos0 + r, KV slot row0 + r
  void* kbase;                 // strided: [Hkv][pitch][D]
  void* vbase;
  int32_t row0, pitch;
  int32_t pos[EPI_MAX_ROWS];
  void* krow[EPI_MAX_ROWS];    // batched: pointer to row slot of head 0; head j at + j * pitch_r * D
  void* vrow[EPI_MAX_ROWS];
  int32_t rpitch[EPI_MAX_ROWS];
};

vc_status epilogue(const EpiArgs& a, hipStream_t s);

}  // namespace vc
