// Internal launch interface of the quantized-cache draft attention (attention_quant.hip).
// Its partials (m, l, o[D]) share the layout and the merge of the other attention kernels.
#pragma once
#include "attention.h"

namespace vc {

// Quantized main region of one request (one layer), plus the per-request
// view of the draft query.
struct QuantSeg {
  const uint8_t* kc;   // [Hkv][Tq][D*b/8]
  const uint8_t* vc;   // [Hkv][Tq/64][D][64*b/8]
  const uint16_t* ks;  // [Hkv][Tq/G][D] fp16
  const uint16_t* kz;
  const uint16_t* vs;  // [Hkv][Tq][D/G] fp16
  const uint16_t* vz;
  int32_t tq;          // quantized rows
  int32_t pad_;
};

// Workgroup y = 0 of a request computes the partial of its exact bf16 rows (the residual
// rows a past the last whole group, then the tail b) into partial slot n_splits; workgroup
// y = s + 1 computes quantized split s into slot s.
struct QuantReq {
  const void* q;       // [1][Hq][D] bf16
  QuantSeg m;
  KVSeg a, b;          // exact rows: residual, then tail (bf16, [Hkv][..][D])
  float* part;         // [1][Hq][s_total][D + 2]
  int32_t s_total, n_splits;
};

struct QuantArgs {
  QuantReq r[VC_MAX_BATCH];
  int32_t n_req, Hq, Hkv, G, bits, group, split_len, max_splits;
  float scale_log2;
};
static_assert(sizeof(QuantArgs) <= 4096, "kernel argument block too large");

// Keys per split of the quantized decode (split_len of QuantArgs, head_dim 128): at most 16
// token groups (2048 keys at group 128, 1024 at group 64), a multiple of 256, and few enough
// groups that the split's scaled query fragments (512 bytes per group per query head) fit in
// QUANT_QP_BYTES of LDS.
constexpr int QUANT_QP_BYTES = 32768;
constexpr int QUANT_MAX_GROUPS = 16;
inline int quant_split_len(int G, int group) {
  int groups = QUANT_QP_BYTES / (512 * G);  // >= 4 for G <= 16
  if (groups > QUANT_MAX_GROUPS) groups = QUANT_MAX_GROUPS;
  return groups * group / 256 * 256;
}

// ev_start / ev_stop (may be null): HIP events that take the kernel's own start and end time.
vc_status launch_attn_quant(const QuantArgs& a, hipStream_t s, hipEvent_t ev_start = nullptr,
                            hipEvent_t ev_stop = nullptr);

}  // namespace vc
