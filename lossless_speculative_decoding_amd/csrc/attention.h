// Internal launch interface of the attention kernels.
//
// Every attention call produces split-K partials (m, l, o[D]) per query row and
// query head, then attn_combine merges them in ascending split order:
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  o = sum_s o_s 2^(m_s - M) / L
// (m is kept in log2 units: scores are pre-multiplied by log2(e) / sqrt(D)).
// Keys are addressed by a logical index t over up to three segments (a, then b,
// then c); splits and 64-key tiles are aligned to t = 0, and query row i (position
// index within the call) sees keys t <= lim0 + i.  For verification the logical
// index is the absolute position (a = the prompt positions, b = the committed
// tail, c = the rows under verification), which makes each row's arithmetic
// independent of the row count.
#pragma once
#include "common.h"

namespace vc {

constexpr int ATT_KT = 64;   // keys per tile
constexpr int ATT_RB = 64;   // query rows (row x GQA head) of one 16-row block in each of a workgroup's 4 waves
constexpr int ATT_MB = 16;   // query rows of one MFMA row block

struct KVSeg {
  const void* k;
  const void* v;
  int64_t hstride;  // elements between consecutive KV heads
  int32_t n;        // rows
  int32_t pad_;
};

// Segment a as the union of rows kept on the device and rows staged from the host:
// position t of tile t / 64 is kept iff bit t % 64 of mask[j][tile]; then it is kept
// row cnt[j][tile] + (kept positions below it in the tile), else staged row
// t - cnt[j][tile] - (kept positions below it).
struct MixSeg {
  const void* k;          // kept rows of the layer, [Hkv][..][D]
  const void* v;
  int64_t hstride;        // elements between consecutive KV heads
  const uint64_t* mask;   // [Hkv][nt]; null: segment a is plain
  const int32_t* cnt;     // [Hkv][nt]
  int32_t nt;
  int32_t pad_;
};

struct AttnReq {
  const void* q;     // [rows][Hq][D]
  KVSeg a, b, c;     // logical keys: a[t], then b[t - a.n], then c[t - a.n - b.n]
  MixSeg mix;        // optional split of segment a (decode attention ignores c and mix)
  float* part;       // [rows][Hq][s_total][D + 2]
  int32_t n_rows;
  int32_t lim0;
  int32_t s_off;     // partial slot of this launch's split 0
  int32_t s_total;
  int32_t n_splits;  // splits of this request in this launch
  int32_t pad_;
};

struct AttnArgs {
  AttnReq r[VC_MAX_BATCH];
  int32_t n_req, Hq, Hkv, G, split_len, n_rowblocks, max_splits, head_dim;
  float scale_log2;
};
static_assert(sizeof(AttnArgs) <= 4096, "kernel argument block too large");

// Element pointer of key t's K (is_v = false) or V row for KV head j.
template <typename E, int D>
__device__ __forceinline__ const E* key_row(const AttnReq& R, int j, int t, bool is_v) {
  if (t < R.a.n) {
    if (R.mix.mask != nullptr) {
      const int64_t tl = int64_t(j) * R.mix.nt + (t >> 6);
      const int o = t & 63;
      const uint64_t m = R.mix.mask[tl];
      const int c = R.mix.cnt[tl];
      // set bits of m below bit o, shifting m itself (a mask (1 << o) - 1 would be loop invariant
      // per lane and get hoisted: one 64-bit register pair per call site)
      const int below = o ? __popcll(m << (64 - o)) : 0;
      if ((m >> o) & 1) {
        const E* base = static_cast<const E*>(is_v ? R.mix.v : R.mix.k);
        return base + j * R.mix.hstride + int64_t(c + below) * D;
      }
      const E* base = static_cast<const E*>(is_v ? R.a.v : R.a.k);
      return base + j * R.a.hstride + int64_t(t - c - below) * D;
    }
    const E* base = static_cast<const E*>(is_v ? R.a.v : R.a.k);
    return base + j * R.a.hstride + int64_t(t) * D;
  }
  t -= R.a.n;
  if (t < R.b.n) {
    const E* base = static_cast<const E*>(is_v ? R.b.v : R.b.k);
    return base + j * R.b.hstride + int64_t(t) * D;
  }
  t -= R.b.n;
  const E* base = static_cast<const E*>(is_v ? R.c.v : R.c.k);
  return base + j * R.c.hstride + int64_t(t) * D;
}

// Address-range check (debug mode) of the rows [0, rows) of every KV head of a segment.
vc_status dbg_kv_seg(const char* kernel, const char* what, const KVSeg& g, int Hkv, int D, int eb, int64_t rows);
// Of one many-row or decode request: queries, segments (with a token-drop split), partials.
vc_status dbg_attn_req(const char* kernel, const AttnReq& R, int Hq, int Hkv, int D, int eb);

// ev_start / ev_stop (may be null) in the launchers below: HIP events that take the
// kernel's own start and end time (hipExtLaunchKernelGGL), for live kernel timing without
// marker-packet gaps; when nothing is launched they are recorded on the stream instead.

// Many-row attention. dtype: VC_BF16 (head_dim 128, MFMA) or VC_F32 (head_dim 64, VALU)
vc_status launch_attn(const AttnArgs& a, int dtype, hipStream_t s, hipEvent_t ev_start = nullptr,
                      hipEvent_t ev_stop = nullptr);

// One-row decode (bf16, head_dim 128, G <= 16): segment a occupies logical keys
// [0, align64(a.n)), segment b follows; lim0 is ignored (every key is visible) and
// split_len must be a multiple of 256.  Logical key count for n_splits:
inline int decode_keys(int a_n, int b_n) { return ((a_n + ATT_KT - 1) / ATT_KT) * ATT_KT + b_n; }
vc_status launch_attn_decode(const AttnArgs& a, hipStream_t s, hipEvent_t ev_start = nullptr,
                             hipEvent_t ev_stop = nullptr);

struct CombineArgs {
  const float* part[VC_MAX_BATCH];  // [rows][Hq][s_total][D+2]
  void* out[VC_MAX_BATCH];          // [rows][Hq][D]
  int32_t s_used[VC_MAX_BATCH];     // slots to merge (<= s_total)
  int32_t n_req, n_rows, Hq, s_total, head_dim, out_dtype;
};
vc_status launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace vc
