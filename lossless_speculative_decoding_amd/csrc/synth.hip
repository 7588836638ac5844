// Seeded synthetic inputs on the GPU (not part of the method).
//
// Counter-based SplitMix64 (Steele, Lea & Flood, OOPSLA 2014; Vigna's
// splitmix64.c): z(c) = mix(c + 0x9E3779B97F4A7C15) with the published
// finaliser, counter c = stream*2^40 + seed*2^32 + index, u = (z >> 40) * 2^-24.
// Draws are evaluated in float64 and rounded float64 -> float32 -> bf16
// (round to nearest even at each step), the same recipe as the host-side
// generator used by the tests, which compare the two bit for bit.
#include "bounds.h"
#include "common.h"

namespace vc {

namespace {

__device__ __forceinline__ uint64_t splitmix64(uint64_t c) {
  uint64_t z = c + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
__device__ __forceinline__ double u24(uint64_t c) { return double(splitmix64(c) >> 40) * (1.0 / 16777216.0); }
__device__ __forceinline__ uint64_t ctr(uint32_t stream, uint32_t seed, uint64_t idx) {
  return (uint64_t(stream) << 40) + (uint64_t(seed) << 32) + idx;
}
__device__ __forceinline__ uint16_t bf16_of_f32(float f) { return f2bf(f); }

__global__ void xavier_kernel(void* dst, int dtype, int64_t n, uint32_t stream, uint32_t seed, int64_t start, double a) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double w = (2.0 * u24(ctr(stream, seed, uint64_t(start + i))) - 1.0) * a;
  const float f = float(w);  // float64 -> float32, nearest even
  if (dtype == VC_BF16) static_cast<uint16_t*>(dst)[i] = bf16_of_f32(f);
  else static_cast<float*>(dst)[i] = f;
}

__global__ void normal_heads_kernel(uint16_t* dst, int64_t n, int H, int rows, int D, uint32_t stream, uint32_t seed,
                                    const int32_t* outl, int n_outl, double outl_scale) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double u1 = u24(ctr(stream, seed, 2 * uint64_t(i)));
  const double u2 = u24(ctr(stream, seed, 2 * uint64_t(i) + 1));
  double x = sqrt(-2.0 * log1p(-u1)) * cos(6.283185307179586 * u2);
  if (outl != nullptr) {
    const int d = int(i % D);
    const int64_t head = i / (int64_t(rows) * D);  // b * H + h
    for (int k = 0; k < n_outl; k++)
      if (outl[head * n_outl + k] == d) x *= outl_scale;
  }
  dst[i] = bf16_of_f32(float(x));
}

__global__ void ids_kernel(int32_t* dst, int64_t n, uint32_t stream, uint32_t seed, uint32_t vocab) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  dst[i] = int32_t((splitmix64(ctr(stream, seed, uint64_t(i))) >> 32) % vocab);
}

__global__ void fill_kernel(void* dst, int dtype, int64_t n, float v) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (dtype == VC_BF16) static_cast<uint16_t*>(dst)[i] = bf16_of_f32(v);
  else static_cast<float*>(dst)[i] = v;
}

}  // namespace

}  // namespace vc

using namespace vc;

extern "C" vc_status vc_synth_xavier(void* dst, int32_t dtype, int64_t n, uint32_t stream, uint32_t seed, int64_t start,
                                     int32_t fan_in, int32_t fan_out, hipStream_t s) {
  VC_REQUIRE(dst != nullptr && n >= 0 && fan_in > 0 && fan_out > 0, VC_ERR_ARG, "vc_synth_xavier: bad arguments");
  VC_REQUIRE(dtype == VC_F32 || dtype == VC_BF16, VC_ERR_ARG, "vc_synth_xavier: bad dtype");
  VC_REQUIRE(seed < 256 && stream < (1u << 24) && start >= 0 && start + n <= (int64_t(1) << 32), VC_ERR_ARG,
             "vc_synth_xavier: counter out of range");
  if (n == 0) return VC_OK;
  VC_DBG_LAUNCH("synth_xavier", {"output", dst, n * (dtype == VC_BF16 ? 2 : 4)});
  const double a = sqrt(6.0 / double(fan_in + fan_out));
  hipLaunchKernelGGL(xavier_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, dst, dtype, n, stream, seed, start, a);
  VC_LAUNCH_CHECK();
  return VC_OK;
}

extern "C" vc_status vc_synth_normal_heads(void* dst, int32_t B, int32_t H, int32_t rows, int32_t D, uint32_t stream,
                                           uint32_t seed, const int32_t* outl, int32_t n_outl, float outl_scale,
                                           hipStream_t s) {
  VC_REQUIRE(dst != nullptr && B > 0 && H > 0 && rows > 0 && D > 0, VC_ERR_ARG, "vc_synth_normal_heads: bad shape");
  const int64_t n = int64_t(B) * H * rows * D;
  VC_REQUIRE(2 * n <= (int64_t(1) << 32) && seed < 256 && stream < (1u << 24), VC_ERR_ARG,
             "vc_synth_normal_heads: counter out of range");
  VC_DBG_LAUNCH("synth_normal_heads", {"output", dst, n * 2},
                {"outlier channels", outl, outl ? int64_t(B) * H * n_outl * 4 : 0});
  hipLaunchKernelGGL(normal_heads_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, static_cast<uint16_t*>(dst), n, H,
                     rows, D, stream, seed, outl, n_outl, double(outl_scale));
  VC_LAUNCH_CHECK();
  return VC_OK;
}

extern "C" vc_status vc_synth_ids(int32_t* dst, int64_t n, uint32_t stream, uint32_t seed, int32_t vocab,
                                  hipStream_t s) {
  VC_REQUIRE(dst != nullptr && n >= 0 && vocab > 0, VC_ERR_ARG, "vc_synth_ids: bad arguments");
  VC_REQUIRE(n <= (int64_t(1) << 32) && seed < 256 && stream < (1u << 24), VC_ERR_ARG, "vc_synth_ids: counter range");
  if (n == 0) return VC_OK;
  VC_DBG_LAUNCH("synth_ids", {"output", dst, n * 4});
  hipLaunchKernelGGL(ids_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, dst, n, stream, seed, uint32_t(vocab));
  VC_LAUNCH_CHECK();
  return VC_OK;
}

extern "C" vc_status vc_synth_fill(void* dst, int32_t dtype, int64_t n, float value, hipStream_t s) {
  VC_REQUIRE(dst != nullptr && n >= 0, VC_ERR_ARG, "vc_synth_fill: bad arguments");
  if (n == 0) return VC_OK;
  VC_DBG_LAUNCH("synth_fill", {"output", dst, n * (dtype == VC_BF16 ? 2 : 4)});
  hipLaunchKernelGGL(fill_kernel, dim3(cdiv(n, 256)), dim3(256), 0, s, dst, dtype, n, value);
  VC_LAUNCH_CHECK();
  return VC_OK;
}
