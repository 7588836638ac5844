// Shared device/host helpers of the VeriCache HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <string>

#include "../../include/vc.h"

namespace vc {

// ---------------------------------------------------------------- host side
void set_error(const char* fmt, ...);
#define VC_REQUIRE(cond, code, ...)        \
  do {                                     \
    if (!(cond)) {                         \
      ::vc::set_error(__VA_ARGS__);        \
      return (code);                       \
    }                                      \
  } while (0)
#define VC_HIP(call)                                                                               \
  do {                                                                                             \
    hipError_t e_ = (call);                                                                        \
    if (e_ != hipSuccess) {                                                                        \
      ::vc::set_error("%s failed: %s (%s:%d)", #call, hipGetErrorString(e_), __FILE__, __LINE__); \
      return VC_ERR_HIP;                                                                           \
    }                                                                                              \
  } while (0)
#define VC_LAUNCH_CHECK() VC_HIP(hipGetLastError())
// a launcher that launches nothing still completes the events it was handed
#define VC_EVENTS_IF_EMPTY(ev_start, ev_stop, s)     \
  do {                                               \
    if (ev_start) VC_HIP(hipEventRecord(ev_start, s)); \
    if (ev_stop) VC_HIP(hipEventRecord(ev_stop, s));   \
  } while (0)

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// ---------------------------------------------------------------- vector types
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 / f16 scalars
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
// float -> bf16 round-to-nearest-even (finite inputs; NaN kept quiet)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) { return uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16); }
// two floats -> packed fp16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
}
// two floats -> fp16 hi pair and fp16 lo pair with a ~= hi + lo (about 22 significant bits).
// a - hi is exact in fp32 (hi is a rounded to fp16), so it is taken in one mixed-precision fma
// per value straight from the packed hi word (v_fma_mix_f32: fp16 source half, fp32 rest)
// instead of converting hi back first.  The results feed a conversion, not an MFMA.
__device__ __forceinline__ void split_h2(float a, float b, uint32_t& hi, uint32_t& lo) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  hi = __builtin_bit_cast(uint32_t, h2{(_Float16)a, (_Float16)b});
  float ra, rb;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(ra) : "v"(hi), "v"(a));
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(rb) : "v"(hi), "v"(b));
  lo = __builtin_bit_cast(uint32_t, h2{(_Float16)ra, (_Float16)rb});
}

// two floats -> bf16 hi pair and bf16 lo pair with a ~= hi + lo (about 17 significant bits):
// hi rounds a to bf16 (nearest even), a - hi is exact in fp32 and lo rounds it.  The empty asm
// keeps the compiler from converting a a second time to rebuild hi's low half.
__device__ __forceinline__ void split_bf2(float a, float b, uint32_t& hi, uint32_t& lo) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  hi = __builtin_bit_cast(uint32_t, b2{(__bf16)a, (__bf16)b});
  asm volatile("" : "+v"(hi));
  const float ra = a - __uint_as_float(hi << 16), rb = b - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, b2{(__bf16)ra, (__bf16)rb});
}

template <typename T>
__device__ __forceinline__ T bitcast(const auto& x) {
  static_assert(sizeof(T) == sizeof(x), "size mismatch");
  return __builtin_bit_cast(T, x);
}

// ---------------------------------------------------------------- cross-lane
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }

// ---------------------------------------------------------------- MFMA wrappers (layouts verified on gfx950)
// 16x16x32: A lane l holds A[l%16][8*(l/16)+e]; B lane l holds B[8*(l/16)+e][l%16];
//           D lane l holds D[4*(l/16)+j][l%16].
__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0, 0);
}
// 32x32x16: A lane l holds A[l%32][8*(l/32)+e]; B lane l holds B[8*(l/32)+e][l%32];
//           D lane l holds D[8*(e/4)+4*(l/32)+e%4][l%32], e = 0..15.
__device__ __forceinline__ f32x16 mfma32_bf16(const u32x4& a, const u32x4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8>(a), bitcast<f16x8>(b), c, 0, 0, 0);
}

// gfx950 LDS transpose read of 16-bit elements (ds_read_b64_tr_b16): every lane addresses an
// 8-byte piece (4 elements); in each group of 16 lanes, lane i receives element i & 3 of the
// pieces of lanes i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12 of its group, in that order.
// p must point into LDS and be 8-byte aligned.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const lds_s4* q = (const lds_s4*)((const __attribute__((address_space(3))) uint8_t*)p);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s4*>(q)));
}

// 16-byte load marked non-temporal (streamed once, not kept in the caches)
__device__ __forceinline__ u32x4 ld_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// dword 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle)
constexpr int BUF_DWORD3 = 0x00020000;
// 16-byte buffer load at byte offset off (range-checked against the resource: out of
// range reads as zero), marked non-temporal
__device__ __forceinline__ u32x4 ld_buf_nt(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_huge_valf();

}  // namespace vc
