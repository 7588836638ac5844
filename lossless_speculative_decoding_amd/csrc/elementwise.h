// Internal launchers of the row-wise kernels.
#pragma once
#include "common.h"

namespace vc {

vc_status k_embed(const void* E, const int32_t* tok, void* h, int M, int d, int V, int dt, hipStream_t s);
vc_status k_rmsnorm(const void* x, const void* g, void* y, int M, int d, float eps, int dt, hipStream_t s);
// h += the S split-K partials P [S][M][d] (the residual epilogue), then y = rmsnorm(h) * g: one
// launch, bitwise the two steps' results; for bf16 rows with d a multiple of 2048 (<= 8192).
bool resid_rmsnorm_ok(int d, int dt);
vc_status k_resid_rmsnorm(const float* P, int S, void* h, const void* g, void* y, int M, int d, float eps, int dt,
                          hipStream_t s);
vc_status k_argmax(const float* logits, int M, int V, int32_t* out, hipStream_t s);
vc_status k_accept(int32_t* rows, const int32_t* verified, int x, int32_t* result, hipStream_t s);
vc_status k_gather_tok(const int32_t* const* src, int n, int32_t* tok, hipStream_t s);
vc_status k_scatter_tok(int32_t* const* dst, int n, const int32_t* out, hipStream_t s);
vc_status k_commit_rows(const void* vk, const void* vv, int vcap, void* tk, void* tv, int tcap, int n_tail,
                        int row_bytes, int n_lh, int max_rows, const int32_t* result, hipStream_t s);
vc_status k_rope_table(float* tab, int max_pos, int D, double theta, hipStream_t s);
vc_status k_copy_words(const void* src, void* dst, int64_t bytes, hipStream_t s);

}  // namespace vc
