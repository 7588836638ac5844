// Internal launchers of sampled decoding (sampling.hip).
#pragma once
#include "common.h"

namespace vc {

constexpr int SAMPLE_MAX_ROWS = 16;  // rows per sampling launch

// One row to draw from: logits [V] fp32, the draw's key and counter, where the token goes and
// (optionally) where the row's distribution goes.
struct SampleRow {
  const float* logits;
  float* probs;  // [V] or null
  int32_t* out;
  uint64_t seed, stream;
  int64_t pos;
  float tau;
};

vc_status k_sample(const SampleRow* rows, int n, int V, int purpose, hipStream_t s);
// Speculative rejection sampling of one verified round (see vc_spec_sample); ws: at least
// spec_ws_bytes(x) bytes.
size_t spec_ws_bytes(int x);
vc_status k_spec(const float* logits_t, const float* probs_d, const int32_t* draft, int x, int V, float tau,
                 uint64_t seed, uint64_t stream, int64_t pos0, int32_t* verified, void* ws, hipStream_t s);

}  // namespace vc
