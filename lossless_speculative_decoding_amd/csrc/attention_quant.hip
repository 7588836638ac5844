// Draft-step decode attention over a per-group quantized KV cache (2/3/4-bit).
//
// One workgroup = 4 waves = (request, KV head, split); wave w streams the 64-key tiles
// w, w + 4, ... of the split with its own online softmax, and the four states are merged
// in wave order at the end.  The codes are not staged through LDS: every lane loads
// exactly the packed codes its MFMA fragments need and turns them into fp16 operands
// 1 + c 2^(o - 10) by bit placement under the exponent of 1.0 (see "codes -> fp16 MFMA
// operands" below for the offsets o and where the factors and the offset 1 go).  The
// quantization scale and zero are never applied to the codes; they are folded into
// the other operand instead:
//     q . k_t       = sum_d (q_d s_gd) c_td + sum_d q_d z_gd        (K: scale/zero per channel and token group)
//     sum_t p_t v_t = sum_t (p_t s_t) c_t  + sum_t p_t z_t          (V: scale/zero per token and channel group)
// so the MFMA operands are Q' = q*s, the codes, and P' = p*s (scaled by 2^10 to stay
// out of the fp16 subnormal range).  Codes count as centred (c - 2^(b-1); the zero moves
// to z + 2^(b-1) s) so that the folded sums do not cancel against a large zero term; the
// centring and the conversion's offset 1 are removed by bias terms (K) and by a constant
// "centre row" MFMA after each code MFMA (V), never by arithmetic on the codes.  Q' is
// carried as an fp16 hi/lo pair (two MFMAs, about 22 significant bits: a score error
// moves every weight through the exponential); P' as one fp16 number.
//
// Operand assignment.  Lane l (g = l / 16, r = l % 16) holds for S^T = C_K Q'^T the
// K codes of channels [32g, 32g + 32) of key 16 (r / 4) + 4 kt + r % 4 of the tile
// (16-key block kt): one contiguous 4*BITS-byte piece of a code row, so a wave reads
// whole rows.  The score accumulator of lane (g, head r) then holds keys
// [16g, 16g + 16), which are exactly the keys whose V codes the lane loads for
// O^T += C_V^T P'^T: the 16-code run of channel 16 dt + r starting at token 16g (one
// contiguous 2*BITS-byte piece of a per-channel code row).  The conversion tables below
// fix which code each fp16 position carries (4-bit: [0,4,1,5,2,6,3,7] per 8 codes; 2-bit:
// [0,8,1,9,...,7,15] per 16; 3-bit: its own table); Q' and P' are built in that order.
#include <type_traits>

#include "attention_quant.h"
#include "bounds.h"

namespace vc {

namespace {

constexpr int D = 128;
// ---------------------------------------------------------------- codes -> fp16 MFMA operands
// An output word carries two codes of a lane's run as fp16 numbers 1 + c 2^(o - 10): the b code
// bits sit at mantissa bits [o, o + b) under the exponent of 1.0 (0x3C00), one code per 16-bit
// half.  Word m of a run takes the run's little-endian bit stream from bit s (nothing, one shift
// or one funnel shift of two packed words), keeps the two fields and ors in the exponents: one
// v_and_or_b32 plus at most one shift per word, and words with the same s share the shift.
// Position p = 2m + h of a run's fp16 sequence (h = 0 the low half) holds code lo (h = 0) or
// hi (h = 1) of word m.  The factor 2^(10 - o) of each position goes into the other operand
// (Q' on the K side, the V scale on the V side), and the offset 1 into a bias, so the codes are
// never centred by arithmetic.  The fp32 accumulators then also carry the offsets, 2^(10 - o)
// times the code part at most, and for a diffuse attention row the output is far smaller than
// the weighted sum of offsets: positions keep o >= 4 (3-bit V: o >= 3), which holds the extra
// accumulation error to ~1e-4 of the output (o = 0 measured ~3e-3 at 2k keys).
struct ConvWord {
  int s;         // stream bit that lands at bit 0 (negative: shifted left)
  int lo, olo;   // code index in the run and mantissa offset, low half
  int hi, ohi;   // same, high half
};

template <int BITS> struct KConv;  // K runs: 32 codes (one key, 32 channels), 16 words
template <int BITS> struct VConv;  // V runs: 16 codes (one channel, 16 tokens), 8 words

#define RUN4(w) ConvWord{32 * w - 4, 8 * w, 4, 8 * w + 4, 4}, ConvWord{32 * w, 8 * w + 1, 4, 8 * w + 5, 4}, \
               ConvWord{32 * w + 4, 8 * w + 2, 4, 8 * w + 6, 4}, ConvWord{32 * w + 8, 8 * w + 3, 4, 8 * w + 7, 4}
template <> struct KConv<4> { static constexpr ConvWord w[16] = {RUN4(0), RUN4(1), RUN4(2), RUN4(3)}; };
template <> struct VConv<4> { static constexpr ConvWord w[8] = {RUN4(0), RUN4(1)}; };
#define RUN2(w) ConvWord{32 * w - 4, 16 * w, 4, 16 * w + 8, 4}, ConvWord{32 * w - 4, 16 * w + 1, 6, 16 * w + 9, 6},       \
               ConvWord{32 * w, 16 * w + 2, 4, 16 * w + 10, 4}, ConvWord{32 * w, 16 * w + 3, 6, 16 * w + 11, 6},        \
               ConvWord{32 * w, 16 * w + 4, 8, 16 * w + 12, 8}, ConvWord{32 * w + 6, 16 * w + 5, 4, 16 * w + 13, 4}, \
               ConvWord{32 * w + 6, 16 * w + 6, 6, 16 * w + 14, 6}, ConvWord{32 * w + 6, 16 * w + 7, 8, 16 * w + 15, 8}
template <> struct KConv<2> { static constexpr ConvWord w[16] = {RUN2(0), RUN2(1)}; };
template <> struct VConv<2> { static constexpr ConvWord w[8] = {RUN2(0)}; };
#undef RUN2
#undef RUN4
// 3-bit fields sit at multiples of 3, so the two codes of a word are 5 or 6 apart in the run and
// most words need their own (funnel) shift
template <> struct KConv<3> {
  static constexpr ConvWord w[16] = {{-7, 0, 7, 5, 6},   {-4, 1, 7, 6, 6},   {0, 2, 6, 7, 5},    {2, 3, 7, 8, 6},
                                     {5, 4, 7, 9, 6},    {23, 10, 7, 15, 6}, {26, 11, 7, 16, 6}, {29, 12, 7, 17, 6},
                                     {32, 13, 7, 18, 6}, {35, 14, 7, 19, 6}, {53, 20, 7, 25, 6}, {58, 21, 5, 27, 7},
                                     {61, 22, 5, 28, 7}, {64, 23, 5, 29, 7}, {67, 24, 5, 30, 7}, {71, 26, 7, 31, 6}};
};
// (no pairing of 16 3-bit codes keeps every offset >= 4; five positions use o = 3)
template <> struct VConv<3> {
  static constexpr ConvWord w[8] = {{-7, 0, 7, 4, 3}, {-4, 1, 7, 5, 3},  {0, 2, 6, 7, 5},   {2, 3, 7, 8, 6},
                                    {13, 6, 5, 12, 7}, {20, 9, 7, 13, 3}, {23, 10, 7, 14, 3}, {26, 11, 7, 15, 3}};
};

// every code of the run exactly once, each field where the word's shift puts it
template <int BITS, int N, int OMIN>
constexpr bool conv_table_ok(const ConvWord (&t)[N]) {
  int seen[2 * N] = {};
  for (int m = 0; m < N; m++) {
    const ConvWord& c = t[m];
    if (c.lo < 0 || c.hi < 0 || c.lo >= 2 * N || c.hi >= 2 * N) return false;
    seen[c.lo]++;
    seen[c.hi]++;
    if (BITS * c.lo - c.s != c.olo || BITS * c.hi - c.s - 16 != c.ohi) return false;
    if (c.olo < OMIN || c.ohi < OMIN || c.olo + BITS > 10 || c.ohi + BITS > 10) return false;
  }
  for (int i = 0; i < 2 * N; i++)
    if (seen[i] != 1) return false;
  return true;
}
static_assert(conv_table_ok<4, 16, 4>(KConv<4>::w) && conv_table_ok<2, 16, 4>(KConv<2>::w) &&
                  conv_table_ok<3, 16, 4>(KConv<3>::w), "K conversion tables");
static_assert(conv_table_ok<4, 8, 4>(VConv<4>::w) && conv_table_ok<2, 8, 4>(VConv<2>::w) &&
                  conv_table_ok<3, 8, 3>(VConv<3>::w), "V conversion tables");

// the stream bits of word CW's two fields, shifted so that stream bit CW.s is bit 0
template <int BITS, ConvWord CW, int NW>
__device__ __forceinline__ uint32_t run_bits(const uint32_t (&w)[NW]) {
  constexpr int b0 = BITS * CW.lo, b1 = BITS * CW.hi + BITS - 1;  // first and last bit of the fields
  constexpr int k0 = b0 / 32, k1 = b1 / 32;
  static_assert(k1 < NW, "field past the packed words");
  if constexpr (k0 == k1) {
    constexpr int r = CW.s - 32 * k0;
    if constexpr (r >= 0) return w[k0] >> r;
    else return w[k0] << (-r);
  } else {
    static_assert(k1 == k0 + 1 && CW.s >= 32 * k0 && CW.s < 32 * k0 + 32, "funnel window");
    return __builtin_amdgcn_alignbit(w[k0 + 1], w[k0], CW.s - 32 * k0);
  }
}

template <int BITS, ConvWord CW, int NW>
__device__ __forceinline__ uint32_t conv_word(const uint32_t (&w)[NW]) {
  constexpr uint32_t f = (1u << BITS) - 1;
  constexpr uint32_t mask = (f << CW.olo) | (f << (16 + CW.ohi));
  // (x & mask) | 0x3C003C00 as one v_bitop3_b32 (truth table 0xEA = (a & b) | c); a builtin rather
  // than inline asm, so that the compiler sees the write and keeps the MFMA operand hazards
  return __builtin_amdgcn_bitop3_b32(run_bits<BITS, CW>(w), mask, 0x3C003C00u, 0xEA);
}

// fp16 position p of a run: the code index and mantissa offset it carries
template <typename T>
constexpr int conv_code(int p) { return (p & 1) ? T::w[p >> 1].hi : T::w[p >> 1].lo; }
template <typename T>
constexpr int conv_off(int p) { return (p & 1) ? T::w[p >> 1].ohi : T::w[p >> 1].olo; }
// mantissa offsets of the positions that carry codes 0..15 of a V run, 4 bits each
template <typename T>
constexpr uint64_t conv_offs_by_code() {
  uint64_t r = 0;
  for (int p = 0; p < 16; p++) r |= uint64_t(conv_off<T>(p)) << (4 * conv_code<T>(p));
  return r;
}

template <int BITS>
struct Codes32 {
  uint32_t w[BITS];  // 32 * BITS bits
};

// chunk CH (fp16 positions 8CH .. 8CH + 7) of a K run, built just before its MFMAs
template <int BITS, int CH>
__device__ __forceinline__ u32x4 cvt_k_chunk(const Codes32<BITS>& c) {
  using T = KConv<BITS>;
  return u32x4{conv_word<BITS, T::w[4 * CH]>(c.w), conv_word<BITS, T::w[4 * CH + 1]>(c.w),
               conv_word<BITS, T::w[4 * CH + 2]>(c.w), conv_word<BITS, T::w[4 * CH + 3]>(c.w)};
}

__device__ __forceinline__ float h2f(uint16_t h) { return float(bitcast<_Float16>(h)); }
__device__ __forceinline__ float h2f_lo(uint32_t w) { return h2f(uint16_t(w & 0xffffu)); }
__device__ __forceinline__ float h2f_hi(uint32_t w) { return h2f(uint16_t(w >> 16)); }
// element i of a packed run of 16-bit values held as dwords
__device__ __forceinline__ uint32_t half16(const uint32_t* w, int i) { return (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu); }

// 16 V codes (one channel, 16 consecutive tokens): 2*BITS bytes
template <int BITS>
struct VCodes16 {
  uint32_t w[2];
};

template <int BITS>
__device__ __forceinline__ VCodes16<BITS> ld_vcodes(const uint8_t* src) {
  VCodes16<BITS> c;
  if constexpr (BITS == 2) {
    c.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src));
    c.w[1] = 0;
  } else if constexpr (BITS == 4) {
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
    c.w[0] = x.x;
    c.w[1] = x.y;
  } else {  // 6 bytes at a 2-byte boundary
    const uint16_t* p = reinterpret_cast<const uint16_t*>(src);
    c.w[0] = uint32_t(p[0]) | (uint32_t(p[1]) << 16);
    c.w[1] = p[2];
  }
  return c;
}

// the two chunks (fp16 positions 0..7, 8..15) of a V run
template <int BITS>
__device__ __forceinline__ void cvt_v(const VCodes16<BITS>& c, u32x4 out[2]) {
  using T = VConv<BITS>;
  out[0] = u32x4{conv_word<BITS, T::w[0]>(c.w), conv_word<BITS, T::w[1]>(c.w), conv_word<BITS, T::w[2]>(c.w),
                 conv_word<BITS, T::w[3]>(c.w)};
  out[1] = u32x4{conv_word<BITS, T::w[4]>(c.w), conv_word<BITS, T::w[5]>(c.w), conv_word<BITS, T::w[6]>(c.w),
                 conv_word<BITS, T::w[7]>(c.w)};
}

// The constant "centre row" of the V side, negated: position p holds -W_p with
// W_p = 1 + 2^(b-1) 2^(o_p - 10), so that u - W_p = (c - 2^(b-1)) 2^(o_p - 10) for the code u of
// that position; its fp16 bits are 0xBC00 | 2^(b - 1 + o_p) (exact).  An MFMA of this row with P'
// right after each code MFMA subtracts sum_t P'_t W_t, from the same rounded P', in the same
// accumulator: the accumulators never carry more than one chunk's offsets (the MFMA accumulation
// of large offsets measured ~3e-3 of the output at o = 4 when they were removed only at the end).
template <int BITS>
constexpr uint32_t centre_word(int m) {
  const ConvWord& c = VConv<BITS>::w[m];
  return (0xBC00u | (1u << (BITS - 1 + c.olo))) | ((0xBC00u | (1u << (BITS - 1 + c.ohi))) << 16);
}

template <int BITS>
__device__ __forceinline__ Codes32<BITS> ld_kcodes(const uint8_t* src) {
  Codes32<BITS> c;
  if constexpr (BITS == 4) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
    c.w[0] = x.x; c.w[1] = x.y; c.w[2] = x.z; c.w[3] = x.w;
  } else if constexpr (BITS == 2) {
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
    c.w[0] = x.x; c.w[1] = x.y;
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(src);
    c.w[0] = __builtin_nontemporal_load(p);
    c.w[1] = __builtin_nontemporal_load(p + 1);
    c.w[2] = __builtin_nontemporal_load(p + 2);
  }
  return c;
}

template <int BITS>
__device__ __forceinline__ void ld_ktile(Codes32<BITS> k[4], const uint8_t* kc, int t0, int r16, int g) {
  constexpr int KROW = 16 * BITS;  // bytes per K code row (128 channels)
#pragma unroll
  for (int kt = 0; kt < 4; kt++) {
    const int key = t0 + 16 * (r16 >> 2) + 4 * kt + (r16 & 3);
    k[kt] = ld_kcodes<BITS>(kc + int64_t(key) * KROW + 4 * BITS * g);
  }
}

template <int BITS>
__device__ __forceinline__ void ld_vtile(VCodes16<BITS> v[8], const uint8_t* vc, int t0, int r16, int g) {
  const uint8_t* vb = vc + int64_t(t0 >> 6) * D * (8 * BITS);
#pragma unroll
  for (int dt = 0; dt < 8; dt++) v[dt] = ld_vcodes<BITS>(vb + (16 * dt + r16) * (8 * BITS) + 2 * BITS * g);
}

constexpr int QWAVES = 4;
constexpr int QRED = D + 4;  // floats per head in the merge buffer

// NH: V channel groups per token (1 for group 128, 2 for group 64), a template parameter so
// that every register index below is a compile-time constant.  A split holds at most
// QUANT_MAX_GROUPS token groups: 2048 / NH keys (the LDS tables of the split are sized for it).
template <int NH>
constexpr int qsplit_max() { return QUANT_MAX_GROUPS * D / NH; }

// LDS tables of the split, built once by the whole workgroup before the key loop so that the
// loop reads ready operands:
//   QP  the scaled query Q' = q * s_K of every token group of the split and query head, as the
//       fp16 hi / lo MFMA fragments lanes load directly: u32x4 index
//       ((group * 4 + chunk) * 2 + hi_lo) * 4G + g * G + head (512 bytes per group and head);
//   KB  the key bias sum_d q_d (2^(b-1) s_K + z_K) per token group and head (KBP: its four
//       32-channel partial sums, merged in a fixed order);
//   VF  per key and V channel group: (s_V, 2^(b-1) s_V + z_V) in float32, entry (k, v) at float2
//       k NH + v + k / 16: one 8-byte pad per 16 keys, so that the four 16-key runs the lane
//       groups of a wave read at once fall in different LDS banks (without it they are 128 NH
//       bytes apart: the same banks for NH = 2).
// After the loop the same bytes hold the waves' merge buffer.
template <int NH>
struct QLds {
  static constexpr int QP = 0, KB = QP + QUANT_QP_BYTES, KBP = KB + QUANT_QP_BYTES / 512 * 4,
                       VF = KBP + QUANT_QP_BYTES / 512 * 4 * 4,
                       END = VF + (qsplit_max<NH>() * NH + qsplit_max<NH>() / 16) * 8;
  static constexpr int RED = QWAVES * 16 * QRED * 4;  // also covers the exact rows' 4 * 16 * (D + 2) floats
  static_assert(QWAVES * 16 * (D + 2) * 4 <= RED, "exact-row merge buffer");
  static_assert((16 * D + 4 * 64 * 16) * 4 <= RED, "exact-row query rows and weights");
  static constexpr int BYTES = END > RED ? END : RED;
};

// ---------------------------------------------------------------- exact rows of a request
// The residual and tail rows (bf16, at most a few hundred) of one KV head, for the G query
// heads, on the VALU: wave w takes keys w*64 + lane, w*64 + 256 + lane, ...; the lane of a key
// computes its G scores (query rows from LDS), the wave keeps an online softmax per head, and
// lane l accumulates channels 2l and 2l + 1 of every head.  The four wave states are merged in
// wave order into partial slot `slot`.  lds: at least 4 * G * (D + 2) * 4 bytes (the merge
// buffer, which reuses the query rows' and weights' space).
constexpr int XMAXG = 16;
constexpr int XVB = 16;  // V words loaded together

__device__ __forceinline__ const uint16_t* exact_row(const QuantReq& R, int j, int t, bool is_v) {
  const KVSeg& sg = t < R.a.n ? R.a : R.b;
  const int tt = t < R.a.n ? t : t - R.a.n;
  return static_cast<const uint16_t*>(is_v ? sg.v : sg.k) + j * sg.hstride + int64_t(tt) * D;
}

__device__ void quant_exact_rows(const QuantReq& R, int j, int G, int Hq, float sl2, int slot, uint8_t* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = R.a.n + R.b.n;
  float* qs = reinterpret_cast<float*>(lds);                  // [G][D] query rows, float32
  float* ps = qs + G * D + wave * 64 * G;                       // [64 keys][G] this wave's weights
  float* red = reinterpret_cast<float*>(lds);                   // [4 waves][G][D + 2], after the loop
  for (int i = tid; i < G * D; i += 256)
    qs[i] = bf2f(static_cast<const uint16_t*>(R.q)[int64_t(j * G) * D + i]);
  __syncthreads();
  float m_run[XMAXG], l_run[XMAXG], o0[XMAXG], o1[XMAXG];
#pragma unroll
  for (int h = 0; h < XMAXG; h++) {
    m_run[h] = NEG_INF;
    l_run[h] = 0.f;
    o0[h] = 0.f;
    o1[h] = 0.f;
  }
  for (int t0 = wave * 64; t0 < n; t0 += 256) {
    const int t = t0 + lane;
    const bool ok = t < n;
    // ---- this lane's key: G scores (log2 units)
    float sc[XMAXG];
#pragma unroll
    for (int h = 0; h < XMAXG; h++) sc[h] = 0.f;
    const uint16_t* kr = exact_row(R, j, ok ? t : 0, false);
#pragma unroll 4
    for (int c = 0; c < D / 8; c++) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(kr + 8 * c);
      const float k8[8] = {lo_bf(w.x), hi_bf(w.x), lo_bf(w.y), hi_bf(w.y), lo_bf(w.z), hi_bf(w.z), lo_bf(w.w), hi_bf(w.w)};
#pragma unroll
      for (int h = 0; h < XMAXG; h++) {
        if (h < G) {
#pragma unroll
          for (int e = 0; e < 8; e++) sc[h] = fmaf(qs[h * D + 8 * c + e], k8[e], sc[h]);
        }
      }
    }
    // ---- online softmax per head over the wave's 64 keys
#pragma unroll
    for (int h = 0; h < XMAXG; h++) {
      if (h >= G) continue;  // uniform; keeps the loop fully unrolled (register arrays)
      const float v = ok ? sc[h] * sl2 : NEG_INF;
      float mx = v;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, shfl_xor(mx, o));
      const float m_new = fmaxf(m_run[h], mx);      // finite: lane 0's key of a processed chunk exists
      const float alpha = __builtin_amdgcn_exp2f(m_run[h] - m_new);
      const float pk = __builtin_amdgcn_exp2f(v - m_new);
      float rs = pk;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) rs += shfl_xor(rs, o);
      l_run[h] = l_run[h] * alpha + rs;
      m_run[h] = m_new;
      o0[h] *= alpha;
      o1[h] *= alpha;
      ps[lane * G + h] = pk;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // ---- P.V: lane l accumulates channels 2l, 2l + 1 over the wave's keys, in key order; the
    // V words of XVB keys are loaded together so that their latencies overlap
    const int nk = min(64, n - t0);
    for (int kb = 0; kb < nk; kb += XVB) {
      uint32_t vv[XVB];
#pragma unroll
      for (int k = 0; k < XVB; k++) {
        const int t = t0 + kb + min(k, nk - 1 - kb);  // in range; the excess keys are skipped below
        vv[k] = *reinterpret_cast<const uint32_t*>(exact_row(R, j, t, true) + 2 * lane);
      }
#pragma unroll
      for (int k = 0; k < XVB; k++) {
        if (kb + k < nk) {
          const float v0 = lo_bf(vv[k]), v1 = hi_bf(vv[k]);
#pragma unroll
          for (int h = 0; h < XMAXG; h++) {
            if (h < G) {
              const float p = ps[(kb + k) * G + h];
              o0[h] = fmaf(p, v0, o0[h]);
              o1[h] = fmaf(p, v1, o1[h]);
            }
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  // ---- merge the four wave states in wave order
  __syncthreads();  // every wave is done with the query rows and weights the merge buffer reuses
  float* rw = red + wave * G * (D + 2);
#pragma unroll
  for (int h = 0; h < XMAXG; h++) {
    if (h >= G) continue;
    if (lane == 0) {
      rw[h * (D + 2)] = m_run[h];
      rw[h * (D + 2) + 1] = l_run[h];
    }
    rw[h * (D + 2) + 2 + 2 * lane] = o0[h];
    rw[h * (D + 2) + 2 + 2 * lane + 1] = o1[h];
  }
  __syncthreads();
  for (int idx = tid; idx < G * (D + 2); idx += 256) {
    const int h = idx / (D + 2), e = idx - h * (D + 2);
    float mw[4];
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      mw[w] = red[(w * G + h) * (D + 2)];
      M = fmaxf(M, mw[w]);
    }
    float acc = 0.f;
    if (e == 0) {
      acc = M;
    } else {
#pragma unroll
      for (int w = 0; w < 4; w++) {
        const float wt = mw[w] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
        acc = fmaf(red[(w * G + h) * (D + 2) + e], wt, acc);
      }
    }
    R.part[(int64_t(j * G + h) * R.s_total + slot) * (D + 2) + e] = acc;
  }
}

#ifndef QUANT_WPE2
#define QUANT_WPE2 2
#endif
template <int BITS, int NH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NH == 1 ? 3 : QUANT_WPE2, NH == 1 ? 3 : QUANT_WPE2))) void attn_quant_kernel(
    const QuantArgs args) {
  using L = QLds<NH>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::BYTES];
  u32x4* const s_qp = reinterpret_cast<u32x4*>(lds + L::QP);
  float* const s_kb = reinterpret_cast<float*>(lds + L::KB);
  float* const s_kbp = reinterpret_cast<float*>(lds + L::KBP);
  float* const s_vf = reinterpret_cast<float*>(lds + L::VF);
  float* const red = reinterpret_cast<float*>(lds);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int z = blockIdx.z;
  if (z >= args.n_req) return;
  const QuantReq& R = args.r[z];
  const int G = args.G, Hq = args.Hq;
  const int j = blockIdx.x;
  if (blockIdx.y == 0) {  // the request's exact rows, first in the grid so that they finish early
    quant_exact_rows(R, j, G, Hq, args.scale_log2, R.n_splits, lds);
    return;
  }
  const int s = blockIdx.y - 1;
  if (s >= R.n_splits) return;  // uniform across the workgroup
  const int Tq = R.m.tq;
  const int grp_sz = args.group;
  constexpr bool two = NH == 2;
  constexpr int nh = NH;
  const int ng = Tq / grp_sz;
  const int nblk = Tq / 64;
  const int key_lo = s * args.split_len;
  const int key_hi = min(key_lo + args.split_len, Tq);
  const int r16 = lane & 15, g = lane >> 4;
  const bool head_ok = r16 < G;
  // lanes past the group's heads compute a copy of the last head (finite, never written)
  const int hc = min(r16, G - 1);

  const uint8_t* kc = R.m.kc + int64_t(j) * Tq * (D * BITS / 8);
  const uint8_t* vc = R.m.vc + int64_t(j) * nblk * D * (8 * BITS);
  const uint16_t* ks = R.m.ks + int64_t(j) * ng * D;
  const uint16_t* kz = R.m.kz + int64_t(j) * ng * D;
  const uint16_t* vs = R.m.vs + int64_t(j) * Tq * nh;
  const uint16_t* vz = R.m.vz + int64_t(j) * Tq * nh;
  constexpr float C0 = float(1 << (BITS - 1));
  const int g_lo = key_lo / grp_sz, n_grp = (key_hi - key_lo) / grp_sz;

  // the first tile's codes are in flight while the tables are built
  Codes32<BITS> kr[4];
  VCodes16<BITS> vr[8];
  int t0 = key_lo + ATT_KT * wave;
  if (t0 < key_hi) {
    ld_ktile<BITS>(kr, kc, t0, r16, g);
    ld_vtile<BITS>(vr, vc, t0, r16, g);
  }

  // ---- split tables.  Item (group, head, quarter): channels [32 quarter, +32) of Q' in the
  // lane order of the MFMA fragments (position p carries channel 32 quarter + conv_code(p)),
  //     Q'_p = q s_K 2^(10 - o_p) scale_log2   (scores come out in log2 units),
  // split into fp16 hi + lo, and the quarter's key-bias partial
  //     scale_log2 sum q z_K - sum_p (hi_p + lo_p),
  // which removes the offset 1 of every code from the score using exactly the Q' the MFMAs use.
  using KT = KConv<BITS>;
  const float sl2 = args.scale_log2;
  for (int it = tid; it < n_grp * G * 4; it += 256) {
    const int gi = it / (4 * G), h = (it / 4) % G, qq = it % 4;
    const u32x4* qv = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(R.q) + int64_t(j * G + h) * D + 32 * qq);
    const u32x4* sp = reinterpret_cast<const u32x4*>(ks + int64_t(g_lo + gi) * D + 32 * qq);
    const u32x4* zp = reinterpret_cast<const u32x4*>(kz + int64_t(g_lo + gi) * D + 32 * qq);
    uint32_t sw[16], zw[16], qw[16];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const u32x4 a = sp[i], b = zp[i], c = qv[i];
      sw[4 * i] = a.x; sw[4 * i + 1] = a.y; sw[4 * i + 2] = a.z; sw[4 * i + 3] = a.w;
      zw[4 * i] = b.x; zw[4 * i + 1] = b.y; zw[4 * i + 2] = b.z; zw[4 * i + 3] = b.w;
      qw[4 * i] = c.x; qw[4 * i + 1] = c.y; qw[4 * i + 2] = c.z; qw[4 * i + 3] = c.w;
    }
    float bqz = 0.f, boff = 0.f;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      uint32_t w[4], wl[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; e2++) {
        float pr[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
          const int pos = 8 * c + 2 * e2 + h2;
          const int ch = conv_code<KT>(pos);  // channel 32 qq + ch
          const float qd = (ch & 1) ? hi_bf(qw[ch >> 1]) : lo_bf(qw[ch >> 1]);
          const float sd = h2f(uint16_t(half16(sw, ch))), zd = h2f(uint16_t(half16(zw, ch)));
          bqz = fmaf(qd, zd, bqz);
          pr[h2] = (qd * sd) * (sl2 * float(1 << (10 - conv_off<KT>(pos))));
        }
        // Left to itself the compiler may round the same product to fp16 in two ways (a fused
        // v_fma_mixlo_f16 for one use, the product rounded to fp32 and then converted for
        // another): the hi of the stored word and the hi that lo is taken against could then
        // differ by one ulp, and so could the bias's hi and the MFMAs' (~1e-2 in a score).  Empty
        // asm statements (no instruction) make the fp32 product and the stored words opaque, so
        // hi + lo is the product to 2^-22 and the bias is taken from the very bits the MFMAs read.
        asm volatile("" : "+v"(pr[0]), "+v"(pr[1]));
        split_h2(pr[0], pr[1], w[e2], wl[e2]);
        asm volatile("" : "+v"(w[e2]), "+v"(wl[e2]));
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
          const float hi = h2f(uint16_t(w[e2] >> (16 * h2))), lo = h2f(uint16_t(wl[e2] >> (16 * h2)));
          boff += hi + lo;
        }
      }
      s_qp[((gi * 4 + c) * 2 + 0) * 4 * G + qq * G + h] = u32x4{w[0], w[1], w[2], w[3]};
      s_qp[((gi * 4 + c) * 2 + 1) * 4 * G + qq * G + h] = u32x4{wl[0], wl[1], wl[2], wl[3]};
    }
    s_kbp[it] = fmaf(bqz, sl2, -boff);
  }
  // V scale of key t with the factor 2^(10 - o) of the position that carries it (its index in
  // its 16-token run), and the V bias weight 2^(b-1) s_V + z_V
  using VT = VConv<BITS>;
  for (int i = tid; i < (key_hi - key_lo) * nh; i += 256) {
    const float sv = h2f(vs[int64_t(key_lo) * nh + i]), zv = h2f(vz[int64_t(key_lo) * nh + i]);
    constexpr uint64_t offs = conv_offs_by_code<VT>();
    const int o = int((offs >> (4 * ((i / nh) & 15))) & 15);
    const int e = i + (i / nh >> 4);
    s_vf[2 * e] = sv * float(1 << (10 - o));
    s_vf[2 * e + 1] = fmaf(sv, C0, zv);
  }
  __syncthreads();
  // the four quarter sums of a (group, head) in the order ((0 + 1) + (2 + 3))
  for (int it = tid; it < n_grp * G; it += 256) {
    const float* p4 = s_kbp + 4 * it;
    s_kb[it] = (p4[0] + p4[1]) + (p4[2] + p4[3]);
  }
  __syncthreads();

  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; dt++) oacc[dt] = f32x4{0, 0, 0, 0};
  // the negated centre row as an MFMA operand: the same fp16 positions in every lane
  const u32x4 wcen[2] = {u32x4{centre_word<BITS>(0), centre_word<BITS>(1), centre_word<BITS>(2), centre_word<BITS>(3)},
                         u32x4{centre_word<BITS>(4), centre_word<BITS>(5), centre_word<BITS>(6), centre_word<BITS>(7)}};
  float vb0 = 0.f, vb1 = 0.f;
  float m_run = NEG_INF, l_run = 0.f;

  for (; t0 < key_hi; t0 += QWAVES * ATT_KT) {
    // V scale (times the factor of the key's position) and bias weight of this lane's keys
    // [t0 + 16g, t0 + 16g + 16): key k, channel group v at vf[k * NH + v]
    const int run0 = t0 - key_lo + 16 * g;
    const float2* const vf = reinterpret_cast<const float2*>(s_vf) + run0 * nh + (run0 >> 4);
    // ---- key bias of the tile's token group; its Q' fragments are read per 32-channel chunk
    // (holding them across tiles, or all four chunks at once, would keep registers live)
    const int gi = t0 / grp_sz - g_lo;
    const float kbias = s_kb[gi * G + hc];
    const u32x4* const qp = s_qp + (gi * 4 * 2) * 4 * G + g * G + hc;

    // ---- S^T = C_K Q'^T: lane (g, head r) gets keys 16g + 4kt + jj; chunk-outer, so the four
    // 16-key blocks are independent MFMA chains
    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; kt++) sacc[kt] = f32x4{0, 0, 0, 0};
    auto s_chunk = [&](auto chv) {
      constexpr int c = decltype(chv)::value;
      const u32x4 qh = qp[(c * 2 + 0) * 4 * G], ql = qp[(c * 2 + 1) * 4 * G];
#pragma unroll
      for (int kt = 0; kt < 4; kt++) {
        const u32x4 ka = cvt_k_chunk<BITS, c>(kr[kt]);
        sacc[kt] = mfma_f16(ka, qh, sacc[kt]);
        sacc[kt] = mfma_f16(ka, ql, sacc[kt]);
      }
    };
    s_chunk(std::integral_constant<int, 0>{});
    s_chunk(std::integral_constant<int, 1>{});
    s_chunk(std::integral_constant<int, 2>{});
    s_chunk(std::integral_constant<int, 3>{});
    // the next tile's K codes are in flight during the softmax and P.V of this one
    const int tn = t0 + QWAVES * ATT_KT;
    if (tn < key_hi) ld_ktile<BITS>(kr, kc, tn, r16, g);

    // ---- online softmax per head (every key of a tile is visible), in log2 units: the score of a
    // key is its MFMA sum plus the group's key bias, p = 2^(score - m).
    float mx = NEG_INF;
#pragma unroll
    for (int kt = 0; kt < 4; kt++)
      mx = fmaxf(mx, fmaxf(fmaxf(sacc[kt][0], sacc[kt][1]), fmaxf(sacc[kt][2], sacc[kt][3])));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx + kbias);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float nb = kbias - m_new;
    float rs = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; kt++) {
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const float p = __builtin_amdgcn_exp2f(sacc[kt][jj] + nb);
        sacc[kt][jj] = p;
        rs += p;
      }
    }
    rs += shfl_xor(rs, 16);
    rs += shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__any(alpha != 1.f)) {  // the running max rarely moves after the first tiles; x * 1 == x
#pragma unroll
      for (int dt = 0; dt < 8; dt++) oacc[dt] *= alpha;
      vb0 *= alpha;
      vb1 *= alpha;
    }

    // ---- P' = p s_V 2^(10 - o) (per V channel group) as one fp16 number, in the V conversion
    // order, and the V bias sum p (2^(b-1) s_V + z_V).  With the centre row, the output is
    //     sum_t P'_t (u_t - W_t) + bias = sum_t P'_t (c_t - 2^(b-1)) 2^(o-10) + bias,
    // so one fp16 rounding of each weight (2^-12 relative, independent) meets the centred code,
    // as if the codes had been centred: up to ~6e-4 relative in the output (measured), against
    // ~1e-5 with an fp16 hi/lo pair, for half the P.V MFMAs and P' work.
    u32x4 pb[2][NH];  // [32-key chunk][V channel group]
#pragma unroll
    for (int kc2 = 0; kc2 < 2; kc2++) {
      uint32_t w[NH][4];
#pragma unroll
      for (int e2 = 0; e2 < 4; e2++) {
        float pr[NH][2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int k = conv_code<VT>(8 * kc2 + 2 * e2 + h);  // key 16g + k
          const float x = sacc[k >> 2][k & 3];                // p
#pragma unroll
          for (int v = 0; v < NH; v++) {
            const float2 f = vf[k * NH + v];
            pr[v][h] = x * f.x;
            if (v == 0) vb0 = fmaf(x, f.y, vb0);
            else vb1 = fmaf(x, f.y, vb1);
          }
        }
#pragma unroll
        for (int v = 0; v < NH; v++) w[v][e2] = pack_h2(pr[v][0], pr[v][1]);
      }
#pragma unroll
      for (int v = 0; v < NH; v++) pb[kc2][v] = u32x4{w[v][0], w[v][1], w[v][2], w[v][3]};
    }
    // ---- O^T += C_V^T P'^T (channels 64..127 use the second V group's P' when the group is 64)
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      u32x4 va[2];
      cvt_v<BITS>(vr[dt], va);
      const int v = NH == 2 ? (dt >> 2) : 0;
#pragma unroll
      for (int kc2 = 0; kc2 < 2; kc2++) {
        oacc[dt] = mfma_f16(va[kc2], pb[kc2][v], oacc[dt]);
        oacc[dt] = mfma_f16(wcen[kc2], pb[kc2][v], oacc[dt]);
      }
    }
    if (tn < key_hi) ld_vtile<BITS>(vr, vc, tn, r16, g);
  }

  __syncthreads();  // every wave is done with the scale copies that the merge buffer overwrites
  // ---- this wave's state -> LDS; lane holds o[16dt + 4g + jj] of head l % 16
  vb0 += shfl_xor(vb0, 16);
  vb0 += shfl_xor(vb0, 32);
  vb1 += shfl_xor(vb1, 16);
  vb1 += shfl_xor(vb1, 32);
  if (!two) vb1 = vb0;
  float* rw = red + wave * 16 * QRED;
  if (head_ok) {
    float* rh = rw + r16 * QRED;
    if (g == 0) {
      rh[0] = m_run;
      rh[1] = l_run;
    }
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      const float vbias = dt >= 4 ? vb1 : vb0;
#pragma unroll
      for (int jj = 0; jj < 4; jj++) rh[2 + 16 * dt + 4 * g + jj] = oacc[dt][jj] + vbias;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * (D + 2); idx += 256) {
    const int n = idx / (D + 2), e = idx - n * (D + 2);
    float mw[QWAVES];
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < QWAVES; w++) {
      mw[w] = red[(w * 16 + n) * QRED];
      M = fmaxf(M, mw[w]);
    }
    float acc = 0.f;
    if (e == 0) {
      acc = M;
    } else {
#pragma unroll
      for (int w = 0; w < QWAVES; w++) {
        const float wt = mw[w] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
        acc = fmaf(red[(w * 16 + n) * QRED + e], wt, acc);
      }
    }
    R.part[(int64_t(j * G + n) * R.s_total + s) * (D + 2) + e] = acc;
  }
}

}  // namespace

vc_status launch_attn_quant(const QuantArgs& a, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (a.n_req <= 0) {
    VC_EVENTS_IF_EMPTY(ev_start, ev_stop, s);
    return VC_OK;
  }
  VC_REQUIRE(a.group == 64 || a.group == 128, VC_ERR_UNSUPPORTED, "quant group must be 64 or 128");
  VC_REQUIRE(a.G <= XMAXG, VC_ERR_UNSUPPORTED, "GQA group > %d", XMAXG);
  VC_REQUIRE(a.split_len % (QWAVES * ATT_KT) == 0 && a.split_len % a.group == 0 &&
                 a.split_len / a.group <= QUANT_MAX_GROUPS && (a.split_len / a.group) * a.G * 512 <= QUANT_QP_BYTES,
             VC_ERR_ARG, "quantized decode: split %d must be a multiple of 256 and of the group, hold at most %d "
             "token groups and at most %d token groups x query heads", a.split_len, QUANT_MAX_GROUPS,
             QUANT_QP_BYTES / 512);
  for (int r = 0; r < a.n_req; r++)
    VC_REQUIRE(a.r[r].m.tq % 64 == 0 && a.r[r].m.tq % a.group == 0, VC_ERR_ARG, "quantized rows not whole groups");
  if (dbg_on()) {
    for (int r = 0; r < a.n_req; r++) {
      const QuantReq& q = a.r[r];
      const int64_t tq = q.m.tq, cb = int64_t(a.Hkv) * tq * D * a.bits / 8;
      const int64_t kzb = int64_t(a.Hkv) * (tq / a.group) * D * 2, vzb = int64_t(a.Hkv) * tq * (D / a.group) * 2;
      // quantized splits s < n_splits cover keys [s split_len, min((s + 1) split_len, tq)); the exact
      // rows go to slot n_splits
      if (int64_t(q.n_splits) * a.split_len < tq || q.n_splits + 1 > q.s_total || q.n_splits > a.max_splits)
        return dbg_fail("attn_quant: request %d has %d splits of %d keys for %lld rows, %d slots", r, q.n_splits,
                        a.split_len, (long long)tq, q.s_total);
      if (vc_status st = dbg_check("attn_quant", {{"query", q.q, int64_t(a.Hq) * D * 2},
                                                  {"K codes", q.m.kc, cb}, {"V codes", q.m.vc, cb},
                                                  {"K scales", q.m.ks, kzb}, {"K zeros", q.m.kz, kzb},
                                                  {"V scales", q.m.vs, vzb}, {"V zeros", q.m.vz, vzb},
                                                  {"partials", q.part, int64_t(a.Hq) * q.s_total * (D + 2) * 4}}))
        return st;
      if (vc_status st = dbg_kv_seg("attn_quant", "residual", q.a, a.Hkv, D, 2, q.a.n)) return st;
      if (vc_status st = dbg_kv_seg("attn_quant", "tail", q.b, a.Hkv, D, 2, q.b.n)) return st;
    }
    if (dbg_dry()) return VC_OK;
  }
  dim3 grid(a.Hkv, a.max_splits + 1, a.n_req);
  const bool g64 = a.group == 64;
  switch (a.bits) {
    case 2:
      if (g64) hipExtLaunchKernelGGL((attn_quant_kernel<2, 2>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, a);
      else hipExtLaunchKernelGGL((attn_quant_kernel<2, 1>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, a);
      break;
    case 3:
      if (g64) hipExtLaunchKernelGGL((attn_quant_kernel<3, 2>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, a);
      else hipExtLaunchKernelGGL((attn_quant_kernel<3, 1>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, a);
      break;
    case 4:
      if (g64) hipExtLaunchKernelGGL((attn_quant_kernel<4, 2>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, a);
      else hipExtLaunchKernelGGL((attn_quant_kernel<4, 1>), grid, dim3(256), 0, s, ev_start, ev_stop, 0, a);
      break;
    default: VC_REQUIRE(false, VC_ERR_UNSUPPORTED, "bits must be 2, 3 or 4 (got %d)", a.bits);
  }
  VC_LAUNCH_CHECK();
  return VC_OK;
}

}  // namespace vc
