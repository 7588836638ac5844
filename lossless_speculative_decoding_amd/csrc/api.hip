// C ABI of the VeriCache hot path: model forward for drafting and
// verification, accept / commit, full-KV staging, prefill, compression and
// the single-layer attention entry points.  See include/vc.h for contracts.
#include <algorithm>
#include <cstdarg>
#include <cstring>
#include <functional>
#include <mutex>
#include <vector>

#include "attention.h"
#include "attention_quant.h"
#include "bounds.h"
#include "compress.h"
#include "elementwise.h"
#include "gemm.h"
#include "sampling.h"

namespace vc {

static thread_local std::string g_err;

void set_error(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
}

}  // namespace vc

using namespace vc;

namespace {
// live kernel timing (vc_profile_*): an event pair around a launch (or launch group) of one
// kernel class, with the algorithmic bytes and flops that launch must move and compute
struct ProfRec {
  hipEvent_t a = nullptr, b = nullptr;
  double bytes = 0, flops = 0;
  double aux = 0;  // bytes the launch moves beyond the algorithmic ones (its own split partials)
  int kind = 0;
};
uint32_t g_prof_mask = 0;
std::vector<ProfRec> g_prof[VC_PROF_KINDS];
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence (cache writeback) when the event completes, which would
  // otherwise lengthen the measured interval and the work after it
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// events are null (and nothing is recorded) unless the kind is enabled
ProfRec prof_begin(int kind, double bytes, double flops, double aux = 0) {
  ProfRec r;
  r.kind = kind;
  r.bytes = bytes;
  r.flops = flops;
  r.aux = aux;
  if ((g_prof_mask & (1u << kind)) && !dbg_dry()) {
    r.a = prof_event();
    r.b = prof_event();
    if (!r.a || !r.b) r.a = r.b = nullptr;
  }
  return r;
}

void prof_commit(const ProfRec& r) {
  if (r.a && r.b) g_prof[r.kind].push_back(r);
}

// many-row attention launch: every key visible to the last row read once per KV head (K and V),
// the queries read, the split partials written; flops of QK^T and PV over the causal rows
ProfRec prof_rows(int kind, const AttnArgs& a, int eb) {
  double bytes = 0, flops = 0, aux = 0;
  for (int r = 0; r < a.n_req; r++) {
    const AttnReq& q = a.r[r];
    const double rows = q.n_rows, keys = double(q.lim0) + q.n_rows;
    bytes += double(a.Hkv) * keys * a.head_dim * eb * 2 + rows * a.Hq * a.head_dim * eb;
    aux += rows * a.Hq * q.n_splits * (a.head_dim + 2) * 4.0;
    flops += 4.0 * a.head_dim * a.Hq * (rows * q.lim0 + 0.5 * rows * (rows + 1));
  }
  return prof_begin(kind, bytes, flops, aux);
}

// one projection GEMM: weights + activations read, float32 partials written once
ProfRec prof_gemm(int M, int N, int K, int S, int dtype) {
  const double eb = dtype == VC_BF16 ? 2 : 4;
  const int kind = (dtype == VC_BF16 && M <= 64) ? VC_PROF_GEMM_SKINNY : VC_PROF_GEMM_TILED;
  return prof_begin(kind, (double(N) * K + double(M) * K) * eb, 2.0 * M * N * K, double(S) * M * N * 4);
}
}  // namespace

// File-scope device array behind vc_draft_step_static (see scratch_of_current_device).
static __device__ __align__(256) uint8_t vc_static_scratch[VC_STATIC_SCRATCH_BYTES];

struct vc_model {
  vc_model_desc d;
  vc_weights w;
  float* rope;  // [max_pos][D/2][2]
  int eb;       // bytes per activation / weight element
  // bf16: fragment-major copies of the projection and LM-head weights for the skinny GEMMs
  // (pack_weights), in one allocation; null for fp32 models
  void* wp_mem;
  const void *wp_qkv, *wp_o, *wp_gu, *wp_down, *wp_lm;
};

namespace {

constexpr int SPLIT_VERIFY = 1024;
constexpr int SPLIT_DRAFT = 512;

inline const uint8_t* cptr(const void* p, int64_t off) { return static_cast<const uint8_t*>(p) + off; }
inline uint8_t* mptr(void* p, int64_t off) { return static_cast<uint8_t*>(p) + off; }

// A 2D asynchronous copy, its ranges checked (debug mode) and skipped in dry mode.
vc_status copy2d(const char* what, void* dst, size_t dpitch, const void* src, size_t spitch, size_t width,
                 size_t height, hipMemcpyKind kind, hipStream_t s) {
  if (dbg_on()) {
    if (vc_status st = dbg_check(what, {dbg_2d("destination", dst, dpitch, width, height),
                                        dbg_2d("source", src, spitch, width, height)}))
      return st;
    if (dbg_dry()) return VC_OK;
  }
  VC_HIP(hipMemcpy2DAsync(dst, dpitch, src, spitch, width, height, kind, s));
  return VC_OK;
}

// Device memory the library owns (the RoPE table, temporaries): registered for the range
// checks; lazily mapped host memory in dry mode.
vc_status dev_alloc(void** p, size_t bytes) {
  if (dbg_dry()) {
    *p = dbg_alloc(bytes, false);
    VC_REQUIRE(*p != nullptr, VC_ERR_HIP, "dry run: host allocation of %zu bytes failed", bytes);
    return VC_OK;
  }
  VC_HIP(hipMalloc(p, bytes));
  dbg_register(*p, bytes);
  return VC_OK;
}
void dev_free(void* p) {
  if (!p) return;
  if (dbg_dry()) {
    dbg_free(p, false);
    return;
  }
  dbg_forget(p);
  (void)hipFree(p);
}

struct WsLayout {
  size_t h, a, q, o, m, y, att, tok, total;
};

int64_t n_qkv(const vc_model_desc& d) { return int64_t(d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim; }

size_t gemm_part_bytes(const vc_model_desc& d, int R) {
  const int dt = d.dtype;
  const int64_t Ns[5] = {n_qkv(d), d.d_model, 2 * int64_t(d.ffn), d.d_model, d.vocab};
  const int64_t Ks[5] = {d.d_model, int64_t(d.n_q_heads) * d.head_dim, d.d_model, d.ffn, d.d_model};
  size_t best = 0;
  for (int i = 0; i < 5; i++) {
    const int rs = std::min(R, 64);
    const int S = i == 4 ? 1 : gemm_splits(rs, int(Ns[i]), int(Ks[i]), dt);
    best = std::max(best, size_t(S) * rs * Ns[i] * 4);
    best = std::max(best, size_t(R) * Ns[i] * 4);
  }
  return best;
}

size_t att_part_bytes(const vc_model_desc& d, int R, int max_keys) {
  const int64_t D2 = d.head_dim + 2;
  // quantized splits are shortest for group 64
  const int sq = quant_split_len(d.n_q_heads / d.n_kv_heads, 64);
  const int64_t draft = int64_t(VC_MAX_BATCH) * d.n_q_heads * (cdiv(max_keys, SPLIT_DRAFT) + cdiv(max_keys, sq) + 2) * D2 * 4;
  const int64_t verify = int64_t(R) * d.n_q_heads * (cdiv(max_keys, SPLIT_VERIFY) + 1) * D2 * 4;
  return size_t(std::max(draft, verify));
}

WsLayout ws_layout(const vc_model* m, int R, int max_keys) {
  const vc_model_desc& d = m->d;
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t o = off;
    off = align256(off + b);
    return o;
  };
  const int Rr = std::max(R, VC_MAX_BATCH);
  L.h = take(size_t(Rr) * d.d_model * m->eb);
  L.a = take(size_t(Rr) * d.d_model * m->eb);
  L.q = take(size_t(Rr) * d.n_q_heads * d.head_dim * m->eb);
  L.o = take(size_t(Rr) * d.n_q_heads * d.head_dim * m->eb);
  L.m = take(size_t(Rr) * d.ffn * m->eb);
  L.y = take(gemm_part_bytes(d, Rr));
  L.att = take(att_part_bytes(d, Rr, max_keys));
  L.tok = take(size_t(Rr) * 4 * 2);
  L.total = off;
  return L;
}

// One projection + epilogue.
vc_status proj(const vc_model* m, const void* X, const void* W, const void* Wp, int M, int N, int K, float* P,
               EpiArgs e, hipStream_t s) {
  const int S = gemm_splits(M, N, K, m->d.dtype);
  const ProfRec pr = prof_gemm(M, N, K, S, m->d.dtype);
  vc_status st = gemm(X, W, P, M, N, K, S, m->d.dtype, s, pr.a, pr.b, Wp);
  if (st) return st;
  prof_commit(pr);
  e.P = P;
  e.M = M;
  e.N = N;
  e.S = S;
  e.dtype = m->d.dtype;
  return epilogue(e, s);
}

struct LayerPtrs {
  const uint8_t *wqkv, *wo, *wgu, *wdown, *g1, *g2;
  const uint8_t *pqkv, *po, *pgu, *pdown;  // packed copies (null for fp32 models)
};
LayerPtrs layer_ptrs(const vc_model* m, int l) {
  const vc_model_desc& d = m->d;
  const int64_t eb = m->eb;
  const int64_t dm = d.d_model, hd = int64_t(d.n_q_heads) * d.head_dim;
  LayerPtrs p;
  p.wqkv = cptr(m->w.w_qkv, l * n_qkv(d) * dm * eb);
  p.wo = cptr(m->w.w_o, l * dm * hd * eb);
  p.wgu = cptr(m->w.w_gu, l * 2 * int64_t(d.ffn) * dm * eb);
  p.wdown = cptr(m->w.w_down, l * dm * d.ffn * eb);
  p.g1 = cptr(m->w.norm_attn, l * dm * eb);
  p.g2 = cptr(m->w.norm_ffn, l * dm * eb);
  const bool pk = m->wp_mem != nullptr;
  p.pqkv = pk ? cptr(m->wp_qkv, l * n_qkv(d) * dm * eb) : nullptr;
  p.po = pk ? cptr(m->wp_o, l * dm * hd * eb) : nullptr;
  p.pgu = pk ? cptr(m->wp_gu, l * 2 * int64_t(d.ffn) * dm * eb) : nullptr;
  p.pdown = pk ? cptr(m->wp_down, l * dm * d.ffn * eb) : nullptr;
  return p;
}

// Shared transformer forward over M rows already embedded in ws.h.
vc_status forward_layers(const vc_model* m, int M, uint8_t* ws, const WsLayout& L, EpiArgs qkv_tmpl,
                         const std::function<vc_status(int, EpiArgs&)>& set_kv,
                         const std::function<vc_status(int, const void*, void*, float*)>& attend, hipStream_t s) {
  const vc_model_desc& d = m->d;
  float* P = reinterpret_cast<float*>(ws + L.y);
  void* h = ws + L.h;
  void* a = ws + L.a;
  void* q = ws + L.q;
  void* o = ws + L.o;
  void* mb = ws + L.m;
  const int hd = d.n_q_heads * d.head_dim;
  // weight-streaming rows: a residual projection and the RMSNorm after it run as the GEMM plus one
  // fused residual-and-norm launch (bitwise the epilogue and rmsnorm kernels' results)
  const bool fuse_norm = d.dtype == VC_BF16 && M <= 64 && resid_rmsnorm_ok(d.d_model, d.dtype);
  auto resid_norm = [&](const void* X, const void* W, const void* Wp, int K, const void* gain) -> vc_status {
    const int S = gemm_splits(M, d.d_model, K, d.dtype);
    const ProfRec pr = prof_gemm(M, d.d_model, K, S, d.dtype);
    if (vc_status st1 = gemm(X, W, P, M, d.d_model, K, S, d.dtype, s, pr.a, pr.b, Wp)) return st1;
    prof_commit(pr);
    return k_resid_rmsnorm(P, S, h, gain, a, M, d.d_model, d.eps, d.dtype, s);
  };
  vc_status st;
  for (int l = 0; l < d.n_layers; l++) {
    const LayerPtrs lp = layer_ptrs(m, l);
    if (l == 0 || !fuse_norm) {  // otherwise the previous layer's last projection normalised h already
      if ((st = k_rmsnorm(h, lp.g1, a, M, d.d_model, d.eps, d.dtype, s))) return st;
    }
    EpiArgs e = qkv_tmpl;
    e.mode = EPI_QKV;
    e.q_out = q;
    e.rope = m->rope;
    e.Hq = d.n_q_heads;
    e.Hkv = d.n_kv_heads;
    e.D = d.head_dim;
    if ((st = set_kv(l, e))) return st;
    if ((st = proj(m, a, lp.wqkv, lp.pqkv, M, int(n_qkv(d)), d.d_model, P, e, s))) return st;
    if ((st = attend(l, q, o, reinterpret_cast<float*>(ws + L.att)))) return st;
    if (fuse_norm) {
      if ((st = resid_norm(o, lp.wo, lp.po, hd, lp.g2))) return st;
    } else {
      EpiArgs r{};
      r.mode = EPI_RESID;
      r.out = h;
      if ((st = proj(m, o, lp.wo, lp.po, M, d.d_model, hd, P, r, s))) return st;
      if ((st = k_rmsnorm(h, lp.g2, a, M, d.d_model, d.eps, d.dtype, s))) return st;
    }
    EpiArgs g{};
    g.mode = EPI_SWIGLU;
    g.out = mb;
    if ((st = proj(m, a, lp.wgu, lp.pgu, M, 2 * d.ffn, d.d_model, P, g, s))) return st;
    if (fuse_norm && l + 1 < d.n_layers) {  // the next layer's input norm
      if ((st = resid_norm(mb, lp.wdown, lp.pdown, d.ffn, layer_ptrs(m, l + 1).g1))) return st;
    } else {
      EpiArgs r2{};
      r2.mode = EPI_RESID;
      r2.out = h;
      if ((st = proj(m, mb, lp.wdown, lp.pdown, M, d.d_model, d.ffn, P, r2, s))) return st;
    }
  }
  return VC_OK;
}

// Final norm + LM head of rows [r0, r0 + M) of ws.h, then the argmax of each row or, with smp
// (M rows; their logits and out fields are set here), a draw of the given purpose.
vc_status head(const vc_model* m, int r0, int M, uint8_t* ws, const WsLayout& L, int32_t* out_tok, float* logits_opt,
               hipStream_t s, const SampleRow* smp = nullptr, int purpose = VC_DRAW_TARGET) {
  const vc_model_desc& d = m->d;
  vc_status st;
  const void* hrow = ws + L.h + size_t(r0) * d.d_model * m->eb;
  void* a = ws + L.a;
  float* P = reinterpret_cast<float*>(ws + L.y);
  if ((st = k_rmsnorm(hrow, m->w.norm_final, a, M, d.d_model, d.eps, d.dtype, s))) return st;
  const ProfRec pr = prof_gemm(M, d.vocab, d.d_model, 1, d.dtype);
  if ((st = gemm(a, m->w.lm_head, P, M, d.vocab, d.d_model, 1, d.dtype, s, pr.a, pr.b, m->wp_lm))) return st;
  prof_commit(pr);
  if (smp) {
    SampleRow rows[SAMPLE_MAX_ROWS];
    VC_REQUIRE(M <= SAMPLE_MAX_ROWS, VC_ERR_ARG, "sampled head: %d rows", M);
    for (int r = 0; r < M; r++) {
      rows[r] = smp[r];
      rows[r].logits = P + int64_t(r) * d.vocab;
      rows[r].out = out_tok + r;
    }
    if ((st = k_sample(rows, M, d.vocab, purpose, s))) return st;
  } else if ((st = k_argmax(P, M, d.vocab, out_tok, s))) {
    return st;
  }
  if (logits_opt) {
    const int64_t bytes = int64_t(M) * d.vocab * 4;
    if (dbg_on()) {
      if ((st = dbg_check("logits copy", {{"destination", logits_opt, bytes}, {"source", P, bytes}}))) return st;
      if (dbg_dry()) return VC_OK;
    }
    VC_HIP(hipMemcpyAsync(logits_opt, P, size_t(bytes), hipMemcpyDeviceToDevice, s));
  }
  return VC_OK;
}

vc_status check_model(const vc_model* m) {
  VC_REQUIRE(m != nullptr, VC_ERR_ARG, "null model");
  return VC_OK;
}

// Per-layer views into a compressed blob of L layers.
struct CompView {
  vc_compress_layout lay;
  int kind, bits, group, tq, kk, n_resid, Hkv, D, eb;
  const uint8_t* base;
  KVSeg main_bf16(int l) const {  // token drop: kept rows
    const int64_t per = int64_t(Hkv) * kk * D * eb;
    return KVSeg{base + lay.k_main + l * per, base + lay.v_main + l * per, int64_t(kk) * D, kk, 0};
  }
  MixSeg mix(int l) const {  // token drop: the kept / dropped split of the prompt positions
    const int64_t per = int64_t(Hkv) * kk * D * eb;
    const int64_t nt = lay.n_tiles;
    MixSeg m{};
    m.k = base + lay.k_main + l * per;
    m.v = base + lay.v_main + l * per;
    m.hstride = int64_t(kk) * D;
    m.mask = reinterpret_cast<const uint64_t*>(base + lay.keep_mask + l * int64_t(Hkv) * nt * 8);
    m.cnt = reinterpret_cast<const int32_t*>(base + lay.keep_cnt + l * int64_t(Hkv) * nt * 4);
    m.nt = int32_t(nt);
    return m;
  }
  KVSeg resid(int l) const {
    const int64_t per = int64_t(Hkv) * n_resid * D * eb;
    return KVSeg{base + lay.kr + l * per, base + lay.vr + l * per, int64_t(n_resid) * D, n_resid, 0};
  }
  QuantSeg quant(int l) const {
    const int64_t ng = tq / group, nh = D / group;
    QuantSeg q;
    q.kc = base + lay.kc + l * int64_t(Hkv) * tq * D * bits / 8;
    q.vc = base + lay.vc + l * int64_t(Hkv) * tq * D * bits / 8;
    q.ks = reinterpret_cast<const uint16_t*>(base + lay.ks + l * int64_t(Hkv) * ng * D * 2);
    q.kz = reinterpret_cast<const uint16_t*>(base + lay.kz + l * int64_t(Hkv) * ng * D * 2);
    q.vs = reinterpret_cast<const uint16_t*>(base + lay.vs + l * int64_t(Hkv) * tq * nh * 2);
    q.vz = reinterpret_cast<const uint16_t*>(base + lay.vz + l * int64_t(Hkv) * tq * nh * 2);
    q.tq = tq;
    q.pad_ = 0;
    return q;
  }
};

vc_status comp_view(const void* comp, const vc_compress_desc* cd, CompView& v) {
  VC_REQUIRE(comp != nullptr && cd != nullptr, VC_ERR_ARG, "request without compressed cache");
  vc_status st = compress_layout(cd, &v.lay);
  if (st) return st;
  v.kind = cd->kind;
  v.bits = cd->bits;
  v.group = cd->group;
  v.tq = cd->kind == VC_QUANT ? v.lay.n_main : 0;
  v.kk = cd->kind == VC_TOKDROP ? v.lay.n_main : 0;
  v.n_resid = v.lay.n_resid;
  v.Hkv = cd->n_kv_heads;
  v.D = cd->head_dim;
  v.eb = cd->dtype == VC_BF16 ? 2 : 4;
  v.base = static_cast<const uint8_t*>(comp);
  return VC_OK;
}

// Debug mode: the whole buffers a request claims (tails of tail_cap rows per (layer, head), the
// host rows, the token slots, the compressed blob), each measured from its own base pointer so
// that a capacity larger than the allocation is caught even where a neighbouring buffer follows.
// host_rows: also the host arrays, layers [l0, l1) of them (l1 < 0: all layers)
vc_status dbg_request(const char* where, const vc_model* m, const vc_req& q, bool host_rows, int token_rows = 1,
                      int l0 = 0, int l1 = -1) {
  if (!dbg_on()) return VC_OK;
  const vc_model_desc& d = m->d;
  const int64_t per = int64_t(d.n_layers) * d.n_kv_heads * d.head_dim * m->eb;
  vc_status st = dbg_check(where, {{"request tail K", q.tail_k, q.tail_k ? per * q.tail_cap : 0},
                                   {"request tail V", q.tail_v, q.tail_v ? per * q.tail_cap : 0},
                                   {"request token rows", q.rows, q.rows ? int64_t(token_rows) * 4 : 0}});
  if (!st && host_rows) {
    if (l1 < 0) l1 = d.n_layers;
    const int64_t lay = int64_t(d.n_kv_heads) * d.head_dim * m->eb * q.full_cap;  // one layer of a host array
    const int64_t off = int64_t(l0) * lay, len = int64_t(l1 - l0) * lay;
    st = dbg_check(where, {{"request host K rows", q.full_k_host ? cptr(q.full_k_host, off) : nullptr,
                            q.full_k_host ? len : 0},
                           {"request host V rows", q.full_v_host ? cptr(q.full_v_host, off) : nullptr,
                            q.full_v_host ? len : 0}});
  }
  if (!st && q.comp && q.cd) {
    vc_compress_layout lay;
    if ((st = compress_layout(q.cd, &lay))) return st;
    st = dbg_check(where, {{"compressed blob", q.comp, int64_t(lay.total)}});
  }
  return st;
}

// Draft attention for a batch of requests over (compressed main region, exact tail), one layer.
// tail_n[r]: visible tail rows (own row included).
vc_status draft_attention(int Hq, int Hkv, int D, int dtype, int out_dtype, int n, const CompView* views, int l,
                          const KVSeg* tails, const int* tail_n, const void* q, int64_t q_req_stride_bytes, void* o,
                          int64_t o_req_stride_bytes, float* part, hipStream_t s) {
  const int G = Hq / Hkv;
  const float sl2 = LOG2E / sqrtf(float(D));
  // bf16 head_dim 128: the one-row decode kernel, which numbers the exact-row segment's keys
  // from a 64-aligned start (so its split count uses decode_keys).  A quantized request's
  // exact rows (residual + tail) are one more workgroup of the quantized kernel (one slot).
  const bool decode = dtype == VC_BF16 && D == 128 && G <= 16;
  int s_tot = 0;
  int qs_n[VC_MAX_BATCH], ts_n[VC_MAX_BATCH];
  for (int r = 0; r < n; r++) {
    const CompView& v = views[r];
    if (v.kind == VC_QUANT) {
      VC_REQUIRE(D == 128 && dtype == VC_BF16, VC_ERR_UNSUPPORTED, "quantized draft needs bf16, head_dim 128");
      qs_n[r] = int(cdiv(v.tq, quant_split_len(G, v.group)));
      ts_n[r] = 1;
    } else {
      qs_n[r] = 0;
      ts_n[r] = int(cdiv(decode ? decode_keys(v.kk, tail_n[r]) : v.kk + tail_n[r], SPLIT_DRAFT));
    }
    s_tot = std::max(s_tot, qs_n[r] + ts_n[r]);
  }
  const int64_t per_req = int64_t(Hq) * s_tot * (D + 2);
  QuantArgs qa{};
  qa.n_req = 0;
  AttnArgs aa{};
  aa.n_req = 0;
  aa.Hq = Hq;
  aa.Hkv = Hkv;
  aa.G = G;
  aa.split_len = SPLIT_DRAFT;
  aa.head_dim = D;
  aa.scale_log2 = sl2;
  aa.n_rowblocks = 1;
  aa.max_splits = 0;
  int q_bits = 0, q_group = 0;
  for (int r = 0; r < n; r++) {
    const CompView& v = views[r];
    const void* qr_ptr = cptr(q, r * q_req_stride_bytes);
    KVSeg tail = tails[r];
    tail.n = tail_n[r];
    if (v.kind == VC_QUANT) {
      VC_REQUIRE(q_bits == 0 || (q_bits == v.bits && q_group == v.group), VC_ERR_UNSUPPORTED,
                 "one draft batch must share the quantizer settings");
      q_bits = v.bits;
      q_group = v.group;
      QuantReq& qr = qa.r[qa.n_req++];
      qr.q = qr_ptr;
      qr.m = v.quant(l);
      qr.a = v.resid(l);
      qr.b = tail;
      qr.part = part + r * per_req;
      qr.s_total = s_tot;
      qr.n_splits = qs_n[r];
      qa.max_splits = std::max(qa.max_splits, qs_n[r]);
    } else {
      AttnReq& ar = aa.r[aa.n_req++];
      ar.q = qr_ptr;
      ar.part = part + r * per_req;
      ar.n_rows = 1;
      ar.s_total = s_tot;
      ar.a = v.main_bf16(l);
      ar.b = tail;
      ar.lim0 = v.kk + tail_n[r] - 1;
      ar.s_off = 0;
      ar.n_splits = ts_n[r];
      aa.max_splits = std::max(aa.max_splits, ts_n[r]);
    }
  }
  // algorithmic bytes of the partial launches (for vc_profile_read)
  double bytes = 0, flops_keys = 0, aux = 0;  // flops_keys: query heads x keys attended
  for (int r = 0; r < n; r++) {
    const CompView& v = views[r];
    const double row = double(D) * (dtype == VC_BF16 ? 2 : 4);
    if (v.kind == VC_QUANT) {
      const double ng = v.tq / v.group, nh = D / v.group;
      bytes += double(Hkv) * (2.0 * v.tq * D * v.bits / 8 + 2.0 * ng * D * 2 + 2.0 * v.tq * nh * 2);
      bytes += double(Hkv) * (v.n_resid + tail_n[r]) * row * 2;
      flops_keys += double(Hq) * (v.tq + v.n_resid + tail_n[r]);
    } else {
      bytes += double(Hkv) * (v.kk + tail_n[r]) * row * 2;
      flops_keys += double(Hq) * (v.kk + tail_n[r]);
    }
    bytes += double(Hq) * row;                                       // query
    aux += double(Hq) * (qs_n[r] + ts_n[r]) * (D + 2) * 4.0;          // partials written
  }
  // live timing: the first partial launch's own start and the last one's own end
  ProfRec rec = prof_begin(VC_PROF_DRAFT_ATTN, bytes, 4.0 * flops_keys * D, aux);
  vc_status st;
  const bool both = qa.n_req > 0 && aa.n_req > 0;
  if (qa.n_req > 0) {
    qa.Hq = Hq;
    qa.Hkv = Hkv;
    qa.G = G;
    qa.bits = q_bits;
    qa.group = q_group;
    qa.split_len = quant_split_len(G, q_group);
    qa.scale_log2 = sl2;
    if ((st = launch_attn_quant(qa, s, rec.a, both ? nullptr : rec.b))) return st;
  }
  if (aa.n_req > 0) {
    hipEvent_t start = both ? nullptr : rec.a;
    if (decode) {
      if ((st = launch_attn_decode(aa, s, start, rec.b))) return st;
    } else {
      if ((st = launch_attn(aa, dtype, s, start, rec.b))) return st;
    }
  }
  prof_commit(rec);
  CombineArgs c{};
  c.n_req = n;
  c.n_rows = 1;
  c.Hq = Hq;
  c.s_total = s_tot;
  c.head_dim = D;
  c.out_dtype = out_dtype;
  for (int r = 0; r < n; r++) {
    c.part[r] = part + r * per_req;
    c.out[r] = mptr(o, r * o_req_stride_bytes);
    c.s_used[r] = qs_n[r] + ts_n[r];
  }
  return launch_combine(c, s);
}

}  // namespace

// ============================================================================ C ABI
extern "C" {

const char* vc_last_error(void) { return g_err.c_str(); }

vc_status vc_profile_enable(uint32_t mask) {
  g_prof_mask = mask & ((1u << VC_PROF_KINDS) - 1);
  return VC_OK;
}

vc_status vc_profile_read(int32_t kind, vc_profile_stats* out) {
  VC_REQUIRE(out != nullptr, VC_ERR_ARG, "vc_profile_read: null output");
  VC_REQUIRE(kind >= 0 && kind < VC_PROF_KINDS, VC_ERR_ARG, "vc_profile_read: bad kind %d", kind);
  *out = vc_profile_stats{0, 0.0, 0.0, 0.0, 0.0};
  for (ProfRec& r : g_prof[kind]) {
    VC_HIP(hipEventSynchronize(r.b));
    float ms = 0.f;
    VC_HIP(hipEventElapsedTime(&ms, r.a, r.b));
    out->launches += 1;
    out->total_ms += ms;
    out->bytes += r.bytes;
    out->aux_bytes += r.aux;
    out->flops += r.flops;
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof[kind].clear();
  return VC_OK;
}

int32_t vc_abi_version(void) { return 2; }

vc_status vc_model_create(const vc_model_desc* desc, const vc_weights* w, hipStream_t s, vc_model** out) {
  VC_REQUIRE(desc && w && out, VC_ERR_ARG, "vc_model_create: null argument");
  const vc_model_desc& d = *desc;
  VC_REQUIRE(d.n_layers > 0 && d.d_model > 0 && d.n_q_heads > 0 && d.n_kv_heads > 0 && d.ffn > 0 && d.vocab > 0 &&
                 d.max_pos > 0 && d.n_q_heads % d.n_kv_heads == 0,
             VC_ERR_ARG, "vc_model_create: bad shape");
  VC_REQUIRE((d.dtype == VC_BF16 && d.head_dim == 128) || (d.dtype == VC_F32 && d.head_dim == 64),
             VC_ERR_UNSUPPORTED, "vc_model_create: supported are bf16 with head_dim 128 and fp32 with head_dim 64");
  VC_REQUIRE(d.n_q_heads / d.n_kv_heads <= 16, VC_ERR_UNSUPPORTED, "vc_model_create: GQA group > 16");
  VC_REQUIRE(w->embed && w->lm_head && w->norm_final && w->norm_attn && w->norm_ffn && w->w_qkv && w->w_o && w->w_gu &&
                 w->w_down,
             VC_ERR_ARG, "vc_model_create: null weight pointer");
  if (d.dtype == VC_BF16) {
    VC_REQUIRE(d.d_model % 128 == 0 && d.ffn % 128 == 0 && d.vocab % 128 == 0, VC_ERR_UNSUPPORTED,
               "vc_model_create: bf16 path needs d_model, ffn, vocab multiples of 128");
  }
  vc_model* m = new vc_model();
  m->d = d;
  m->w = *w;
  m->eb = d.dtype == VC_BF16 ? 2 : 4;
  void* rope = nullptr;
  if (vc_status st = dev_alloc(&rope, size_t(d.max_pos) * d.head_dim * 4)) {
    delete m;
    return st;
  }
  m->rope = static_cast<float*>(rope);
  m->wp_mem = nullptr;
  m->wp_qkv = m->wp_o = m->wp_gu = m->wp_down = m->wp_lm = nullptr;
  vc_status st = k_rope_table(m->rope, d.max_pos, d.head_dim, double(d.rope_theta), s);
  if (st == VC_OK && d.dtype == VC_BF16) {
    // fragment-major copies for the skinny GEMMs (decode and verification); prefill chunks read
    // the caller's row-major weights through the GEMM library
    const int64_t L = d.n_layers, dm = d.d_model, hd = int64_t(d.n_q_heads) * d.head_dim;
    const int64_t rows[5] = {L * n_qkv(d), L * dm, L * 2 * int64_t(d.ffn), L * dm, d.vocab};
    const int64_t cols[5] = {dm, hd, dm, d.ffn, dm};
    const void* src[5] = {w->w_qkv, w->w_o, w->w_gu, w->w_down, w->lm_head};
    int64_t total = 0;
    for (int i = 0; i < 5; i++) total += rows[i] * cols[i] * 2;
    st = dev_alloc(&m->wp_mem, size_t(total));
    const void** dst[5] = {&m->wp_qkv, &m->wp_o, &m->wp_gu, &m->wp_down, &m->wp_lm};
    int64_t off = 0;
    for (int i = 0; i < 5 && st == VC_OK; i++) {
      void* p = mptr(m->wp_mem, off);
      st = pack_weights(src[i], p, rows[i], int(cols[i]), s);
      *dst[i] = p;
      off += rows[i] * cols[i] * 2;
    }
  }
  if (st == VC_OK && !dbg_dry() && hipStreamSynchronize(s) != hipSuccess) st = VC_ERR_HIP;
  if (st) {
    dev_free(m->rope);
    if (m->wp_mem) dev_free(m->wp_mem);
    delete m;
    return st;
  }
  *out = m;
  return VC_OK;
}

vc_status vc_model_destroy(vc_model* m) {
  if (!m) return VC_OK;
  dev_free(m->rope);
  if (m->wp_mem) dev_free(m->wp_mem);
  delete m;
  return VC_OK;
}

vc_status vc_ws_size(const vc_model* m, int32_t max_rows, int32_t max_keys, size_t* bytes) {
  if (vc_status st = check_model(m)) return st;
  VC_REQUIRE(bytes && max_rows > 0 && max_keys > 0, VC_ERR_ARG, "vc_ws_size: bad arguments");
  *bytes = ws_layout(m, max_rows, max_keys).total;
  return VC_OK;
}

vc_status vc_compress_layout_of(const vc_compress_desc* d, vc_compress_layout* out) { return compress_layout(d, out); }

vc_status vc_compress_size(const vc_compress_desc* d, size_t* out_bytes, size_t* ws_bytes) {
  VC_REQUIRE(out_bytes && ws_bytes, VC_ERR_ARG, "vc_compress_size: null output");
  vc_compress_layout L;
  if (vc_status st = compress_layout(d, &L)) return st;
  *out_bytes = L.total;
  return compress_ws_bytes(d, ws_bytes);
}

vc_status vc_compress(const vc_compress_desc* d, const void* k, const void* v, const void* q_obs, void* out,
                      size_t out_bytes, void* ws, size_t ws_bytes, hipStream_t s) {
  return compress_run(d, k, v, q_obs, out, out_bytes, ws, ws_bytes, s);
}

}  // extern "C"

namespace {
// The batched draft step over a workspace of ws_bytes bytes at ws (a caller's buffer, or the
// static scratch of vc_draft_step_static).
vc_status draft_step_impl(vc_model* m, const vc_req* reqs, int32_t n, float* logits_opt, void* ws, size_t ws_bytes,
                          hipStream_t s, const vc_sampler* smp = nullptr, float* const* probs = nullptr) {
  if (vc_status st = check_model(m)) return st;
  VC_REQUIRE(reqs && ws, VC_ERR_ARG, "vc_draft_step: null argument");
  VC_REQUIRE(n > 0 && n <= VC_MAX_BATCH, VC_ERR_ARG, "vc_draft_step: batch %d not in [1, %d]", n, VC_MAX_BATCH);
  const vc_model_desc& d = m->d;
  int max_keys = 1;
  CompView views[VC_MAX_BATCH];
  KVSeg tails_k[VC_MAX_BATCH];
  int tail_n[VC_MAX_BATCH];
  for (int r = 0; r < n; r++) {
    const vc_req& q = reqs[r];
    if (vc_status st = comp_view(q.comp, q.cd, views[r])) return st;
    VC_REQUIRE(q.cd->n_layers == d.n_layers && q.cd->n_kv_heads == d.n_kv_heads && q.cd->head_dim == d.head_dim &&
                   q.cd->dtype == d.dtype,
               VC_ERR_ARG, "vc_draft_step: request %d compressed with another shape", r);
    VC_REQUIRE(q.tail_k && q.tail_v && q.rows && q.draft_idx >= 0 && q.n_tail >= 0, VC_ERR_ARG,
               "vc_draft_step: bad request %d", r);
    VC_REQUIRE(q.n_tail + q.draft_idx < q.tail_cap, VC_ERR_CAPACITY, "vc_draft_step: tail of request %d is full", r);
    VC_REQUIRE(q.ctx_len + q.draft_idx < d.max_pos, VC_ERR_CAPACITY, "vc_draft_step: position beyond the RoPE table");
    tail_n[r] = q.n_tail + q.draft_idx + 1;
    max_keys = std::max(max_keys, views[r].lay.n_main + views[r].n_resid + tail_n[r]);
    if (vc_status st = dbg_request("vc_draft_step", m, q, false, q.draft_idx + 2)) return st;
  }
  const WsLayout L = ws_layout(m, n, max_keys);
  VC_REQUIRE(ws_bytes >= L.total, VC_ERR_CAPACITY, "vc_draft_step: workspace %zu < %zu bytes", ws_bytes, L.total);
  if (dbg_on())
    if (vc_status st = dbg_check("vc_draft_step", {{"workspace", ws, int64_t(ws_bytes)}})) return st;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  vc_status st;
  int32_t* tok_in = reinterpret_cast<int32_t*>(w8 + L.tok);
  int32_t* tok_out = tok_in + VC_MAX_BATCH;
  const int32_t* src[VC_MAX_BATCH];
  int32_t* dst[VC_MAX_BATCH];
  for (int r = 0; r < n; r++) {
    src[r] = reqs[r].rows + reqs[r].draft_idx;
    dst[r] = reqs[r].rows + reqs[r].draft_idx + 1;
  }
  if ((st = k_gather_tok(src, n, tok_in, s))) return st;
  if ((st = k_embed(m->w.embed, tok_in, w8 + L.h, n, d.d_model, d.vocab, d.dtype, s))) return st;
  EpiArgs tmpl{};
  tmpl.batched = 1;
  for (int r = 0; r < n; r++) tmpl.pos[r] = reqs[r].ctx_len + reqs[r].draft_idx;
  auto set_kv = [&](int l, EpiArgs& e) -> vc_status {
    for (int r = 0; r < n; r++) {
      const vc_req& q = reqs[r];
      const int64_t off = (int64_t(l) * d.n_kv_heads * q.tail_cap + q.n_tail + q.draft_idx) * d.head_dim * m->eb;
      e.krow[r] = mptr(q.tail_k, off);
      e.vrow[r] = mptr(q.tail_v, off);
      e.rpitch[r] = q.tail_cap;
    }
    return VC_OK;
  };
  auto attend = [&](int l, const void* qb, void* ob, float* part) -> vc_status {
    for (int r = 0; r < n; r++) {
      const vc_req& q = reqs[r];
      const int64_t lo = int64_t(l) * d.n_kv_heads * q.tail_cap * d.head_dim * m->eb;
      tails_k[r] = KVSeg{cptr(q.tail_k, lo), cptr(q.tail_v, lo), int64_t(q.tail_cap) * d.head_dim, 0, 0};
    }
    const int64_t qstride = int64_t(d.n_q_heads) * d.head_dim * m->eb;
    return draft_attention(d.n_q_heads, d.n_kv_heads, d.head_dim, d.dtype, d.dtype, n, views, l, tails_k, tail_n, qb,
                           qstride, ob, qstride, part, s);
  };
  if ((st = forward_layers(m, n, w8, L, tmpl, set_kv, attend, s))) return st;
  if (smp) {
    SampleRow rows[VC_MAX_BATCH];
    for (int r = 0; r < n; r++) {
      const vc_req& q = reqs[r];
      rows[r] = SampleRow{nullptr, probs[r] + int64_t(q.draft_idx) * d.vocab, nullptr, smp[r].seed, smp[r].stream,
                          int64_t(q.ctx_len) + q.draft_idx + 1, smp[r].temperature};
    }
    if ((st = head(m, 0, n, w8, L, tok_out, logits_opt, s, rows, VC_DRAW_DRAFT))) return st;
  } else if ((st = head(m, 0, n, w8, L, tok_out, logits_opt, s))) {
    return st;
  }
  return k_scatter_tok(dst, n, tok_out, s);
}

// Workspace of vc_draft_step_static: one array per GPU the library runs on, held until the process
// ends.  Host code never uses the symbol itself as an address (on the host it is a stand-in, not
// device memory): each device's address is taken once with that device current and kept.
std::mutex g_scratch_mu;
void* g_scratch_dev[VC_MAX_DEVICES] = {};

vc_status scratch_of_current_device(void** out) {
  int dev = 0;
  if (!dbg_dry()) VC_HIP(hipGetDevice(&dev));
  VC_REQUIRE(dev >= 0 && dev < VC_MAX_DEVICES, VC_ERR_UNSUPPORTED, "static scratch: device %d beyond %d", dev,
             VC_MAX_DEVICES);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (dbg_dry()) {  // a host stand-in of the array's size
      p = dbg_alloc(VC_STATIC_SCRATCH_BYTES, false);
    } else {
      VC_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(vc_static_scratch)));
      dbg_register(p, VC_STATIC_SCRATCH_BYTES);
    }
    VC_REQUIRE(p != nullptr, VC_ERR_HIP, "static scratch: no device address");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return VC_OK;
}
}  // namespace

extern "C" {

vc_status vc_draft_step(vc_model* m, const vc_req* reqs, int32_t n, float* logits_opt, void* ws, size_t ws_bytes,
                        hipStream_t s) {
  return draft_step_impl(m, reqs, n, logits_opt, ws, ws_bytes, s);
}

vc_status vc_draft_step_sampled(vc_model* m, const vc_req* reqs, int32_t n, const vc_sampler* smp,
                                float* const* probs, float* logits_opt, void* ws, size_t ws_bytes, hipStream_t s) {
  VC_REQUIRE(smp && probs && reqs && n > 0 && n <= VC_MAX_BATCH, VC_ERR_ARG, "vc_draft_step_sampled: null argument");
  for (int r = 0; r < n; r++) {
    VC_REQUIRE(probs[r], VC_ERR_ARG, "vc_draft_step_sampled: null probabilities of request %d", r);
    VC_REQUIRE(smp[r].temperature >= 0.f && smp[r].temperature < __builtin_huge_valf(), VC_ERR_ARG,
               "vc_draft_step_sampled: temperature of request %d not finite and >= 0", r);
  }
  return draft_step_impl(m, reqs, n, logits_opt, ws, ws_bytes, s, smp, probs);
}

vc_status vc_sample(const float* logits, int32_t n_rows, int32_t vocab, const vc_sampler* smp, const int64_t* pos,
                    int32_t purpose, int32_t* out_tok, float* probs_opt, hipStream_t s) {
  VC_REQUIRE(n_rows >= 0 && vocab > 0, VC_ERR_ARG, "vc_sample: %d rows of %d", n_rows, vocab);
  if (n_rows == 0) return VC_OK;
  VC_REQUIRE(logits && smp && pos && out_tok, VC_ERR_ARG, "vc_sample: null argument");
  VC_REQUIRE(purpose >= VC_DRAW_DRAFT && purpose <= VC_DRAW_TARGET, VC_ERR_ARG, "vc_sample: purpose %d", purpose);
  for (int32_t r0 = 0; r0 < n_rows; r0 += SAMPLE_MAX_ROWS) {
    const int n = std::min<int32_t>(SAMPLE_MAX_ROWS, n_rows - r0);
    SampleRow rows[SAMPLE_MAX_ROWS];
    for (int r = 0; r < n; r++) {
      const vc_sampler& q = smp[r0 + r];
      VC_REQUIRE(q.temperature >= 0.f && q.temperature < __builtin_huge_valf(), VC_ERR_ARG,
                 "vc_sample: temperature of row %d not finite and >= 0", r0 + r);
      rows[r] = SampleRow{logits + int64_t(r0 + r) * vocab,
                          probs_opt ? probs_opt + int64_t(r0 + r) * vocab : nullptr,
                          out_tok + r0 + r,
                          q.seed,
                          q.stream,
                          pos[r0 + r],
                          q.temperature};
    }
    if (vc_status st = k_sample(rows, n, vocab, purpose, s)) return st;
  }
  return VC_OK;
}

vc_status vc_spec_ws_size(int32_t x, size_t* bytes) {
  VC_REQUIRE(x >= 0 && bytes, VC_ERR_ARG, "vc_spec_ws_size: bad argument");
  *bytes = spec_ws_bytes(x);
  return VC_OK;
}

vc_status vc_spec_sample(int32_t vocab, const float* logits_t, const float* probs_d, const int32_t* draft, int32_t x,
                         const vc_sampler* smp, int64_t pos0, int32_t* verified, void* ws, size_t ws_bytes,
                         hipStream_t s) {
  VC_REQUIRE(vocab > 0 && x >= 0, VC_ERR_ARG, "vc_spec_sample: vocab %d, x %d", vocab, x);
  VC_REQUIRE(logits_t && smp && verified && ws && (x == 0 || (probs_d && draft)), VC_ERR_ARG,
             "vc_spec_sample: null argument");
  VC_REQUIRE(smp->temperature >= 0.f && smp->temperature < __builtin_huge_valf(), VC_ERR_ARG,
             "vc_spec_sample: temperature not finite and >= 0");
  VC_REQUIRE(ws_bytes >= spec_ws_bytes(x), VC_ERR_CAPACITY, "vc_spec_sample: workspace %zu < %zu bytes", ws_bytes,
             spec_ws_bytes(x));
  return k_spec(logits_t, probs_d, draft, x, vocab, smp->temperature, smp->seed, smp->stream, pos0, verified, ws, s);
}

vc_status vc_draft_step_static(vc_model* m, const vc_req* reqs, int32_t n, float* logits_opt, hipStream_t s) {
  if (vc_status st = check_model(m)) return st;
  VC_REQUIRE(reqs != nullptr && n > 0 && n <= VC_MAX_BATCH, VC_ERR_ARG, "vc_draft_step_static: bad batch");
  void* ws = nullptr;
  if (vc_status st = scratch_of_current_device(&ws)) return st;
  // the workspace this step needs, against the array's fixed size (draft_step_impl checks the
  // requests themselves)
  int max_keys = 1;
  for (int r = 0; r < n; r++) {
    CompView v;
    if (vc_status st = comp_view(reqs[r].comp, reqs[r].cd, v)) return st;
    max_keys = std::max(max_keys, v.lay.n_main + v.n_resid + reqs[r].n_tail + reqs[r].draft_idx + 1);
  }
  const size_t need = ws_layout(m, n, max_keys).total;
  VC_REQUIRE(need <= VC_STATIC_SCRATCH_BYTES, VC_ERR_CAPACITY,
             "vc_draft_step_static: the step needs %zu bytes of workspace, above the static maximum of %zu", need,
             size_t(VC_STATIC_SCRATCH_BYTES));
  return draft_step_impl(m, reqs, n, logits_opt, ws, VC_STATIC_SCRATCH_BYTES, s);
}

// Where a request's full cache lives.  A VeriCache request (comp != NULL) keeps exact rows on
// the device: the kept prompt rows of a token-drop cache and the tail of committed rows;
// the host holds the rest of the prompt (n_host rows per layer and head, compacted in
// position order).  A plain request (comp == NULL) has its whole context on the host.
struct HostPart {
  bool vmode = false;  // VeriCache request
  bool split = false;  // token drop: prompt positions split between kept rows and host rows
  int prompt = 0;      // positions covered by segment a (T, or ctx_len for a plain request)
  int rows = 0;        // rows per (layer, head) held on the host / staged
  CompView view{};
};

vc_status host_part(const vc_model* m, const vc_req* req, HostPart& hp) {
  hp = HostPart{};
  if (req->comp == nullptr) {
    hp.prompt = req->ctx_len;
    hp.rows = req->ctx_len;
    return VC_OK;
  }
  if (vc_status st = comp_view(req->comp, req->cd, hp.view)) return st;
  const vc_compress_desc& cd = *req->cd;
  const vc_model_desc& d = m->d;
  VC_REQUIRE(cd.n_layers == d.n_layers && cd.n_kv_heads == d.n_kv_heads && cd.head_dim == d.head_dim &&
                 cd.dtype == d.dtype,
             VC_ERR_ARG, "request: compressed cache shape differs from the model");
  VC_REQUIRE(req->ctx_len == cd.seq_len + req->n_tail, VC_ERR_ARG,
             "request: ctx_len %d != prompt %d + committed tail %d", req->ctx_len, cd.seq_len, req->n_tail);
  VC_REQUIRE(req->n_tail == 0 || (req->tail_k && req->tail_v), VC_ERR_ARG, "request: tail rows without a tail");
  hp.vmode = true;
  hp.split = cd.kind == VC_TOKDROP;
  hp.prompt = cd.seq_len;
  hp.rows = hp.view.lay.n_host;
  return VC_OK;
}

}  // extern "C"

namespace {
// vc_verify; with layer_ready, layer l's attention waits on the stream for layer_ready[l] first.
vc_status verify_impl(vc_model* m, const vc_req* req, const void* staged_k, const void* staged_v, int32_t staged_cap,
                      const int32_t* tok, int32_t n_rows, int32_t* out_argmax, float* logits_opt, void* vtail_k,
                      void* vtail_v, int32_t vtail_cap, void* ws, size_t ws_bytes, const hipEvent_t* layer_ready,
                      hipStream_t s) {
  if (vc_status st = check_model(m)) return st;
  VC_REQUIRE(req && tok && out_argmax && vtail_k && vtail_v && ws, VC_ERR_ARG, "vc_verify: null argument");
  VC_REQUIRE(n_rows > 0 && n_rows <= 64, VC_ERR_ARG, "vc_verify: n_rows %d not in [1, 64]", n_rows);
  VC_REQUIRE(vtail_cap >= n_rows, VC_ERR_CAPACITY, "vc_verify: vtail capacity %d < %d rows", vtail_cap, n_rows);
  const vc_model_desc& d = m->d;
  const int ctx = req->ctx_len;
  HostPart hp;
  if (vc_status st0 = host_part(m, req, hp)) return st0;
  VC_REQUIRE(ctx >= 0 && (hp.rows == 0 || (staged_k && staged_v && staged_cap >= hp.rows)), VC_ERR_ARG,
             "vc_verify: staged cache smaller than the %d host rows", hp.rows);
  VC_REQUIRE(ctx + n_rows <= d.max_pos, VC_ERR_CAPACITY, "vc_verify: position beyond the RoPE table");
  const WsLayout L = ws_layout(m, n_rows, ctx + n_rows);
  VC_REQUIRE(ws_bytes >= L.total, VC_ERR_CAPACITY, "vc_verify: workspace %zu < %zu bytes", ws_bytes, L.total);
  if (dbg_on()) {
    // the rows touched in each (layer, head) at the buffers' pitches (a caller may pass windows of
    // a larger cache, as full-KV greedy decoding does)
    const int64_t row = int64_t(d.head_dim) * m->eb, lh = int64_t(d.n_layers) * d.n_kv_heads;
    if (vc_status st = dbg_request("vc_verify", m, *req, false)) return st;
    if (vc_status st = dbg_check("vc_verify", {{"workspace", ws, int64_t(ws_bytes)},
                                               dbg_2d("staged K", staged_k, staged_cap * row, hp.rows * row, lh),
                                               dbg_2d("staged V", staged_v, staged_cap * row, hp.rows * row, lh),
                                               dbg_2d("verify K rows", vtail_k, vtail_cap * row, n_rows * row, lh),
                                               dbg_2d("verify V rows", vtail_v, vtail_cap * row, n_rows * row, lh),
                                               {"tokens", tok, int64_t(n_rows) * 4},
                                               {"argmax", out_argmax, int64_t(n_rows) * 4}}))
      return st;
  }
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  vc_status st;
  if ((st = k_embed(m->w.embed, tok, w8 + L.h, n_rows, d.d_model, d.vocab, d.dtype, s))) return st;
  EpiArgs tmpl{};
  tmpl.batched = 0;
  tmpl.pos0 = ctx;
  tmpl.row0 = 0;
  tmpl.pitch = vtail_cap;
  const int64_t Hkv = d.n_kv_heads, D = d.head_dim, eb = m->eb;
  auto set_kv = [&](int l, EpiArgs& e) -> vc_status {
    e.kbase = mptr(vtail_k, l * Hkv * vtail_cap * D * eb);
    e.vbase = mptr(vtail_v, l * Hkv * vtail_cap * D * eb);
    return VC_OK;
  };
  auto attend = [&](int l, const void* qb, void* ob, float* part) -> vc_status {
    if (layer_ready && !dbg_dry()) VC_HIP(hipStreamWaitEvent(s, layer_ready[l], 0));
    AttnArgs a{};
    a.n_req = 1;
    a.Hq = d.n_q_heads;
    a.Hkv = d.n_kv_heads;
    a.G = d.n_q_heads / d.n_kv_heads;
    a.split_len = SPLIT_VERIFY;
    a.head_dim = d.head_dim;
    a.scale_log2 = LOG2E / sqrtf(float(D));
    a.n_rowblocks = int(cdiv(int64_t(n_rows) * a.G, ATT_RB));
    const int S = int(cdiv(ctx + n_rows, SPLIT_VERIFY));
    a.max_splits = S;
    AttnReq& r = a.r[0];
    r.q = qb;
    // keys in position order: prompt (or the whole context of a plain request), committed
    // tail rows, this call's rows; each key is the same bytes whichever buffer holds it
    const KVSeg vt{cptr(vtail_k, l * Hkv * vtail_cap * D * eb), cptr(vtail_v, l * Hkv * vtail_cap * D * eb),
                   int64_t(vtail_cap) * D, n_rows, 0};
    r.a = KVSeg{hp.rows ? cptr(staged_k, l * Hkv * staged_cap * D * eb) : nullptr,
                hp.rows ? cptr(staged_v, l * Hkv * staged_cap * D * eb) : nullptr, int64_t(staged_cap) * D,
                hp.prompt, 0};
    if (hp.split) {
      r.mix = hp.view.mix(l);
      r.b = KVSeg{cptr(req->tail_k, l * Hkv * req->tail_cap * D * eb), cptr(req->tail_v, l * Hkv * req->tail_cap * D * eb),
                  int64_t(req->tail_cap) * D, req->n_tail, 0};
      r.c = vt;
    } else if (hp.vmode) {
      r.b = KVSeg{cptr(req->tail_k, l * Hkv * req->tail_cap * D * eb), cptr(req->tail_v, l * Hkv * req->tail_cap * D * eb),
                  int64_t(req->tail_cap) * D, req->n_tail, 0};
      r.c = vt;
    } else {
      r.b = vt;
    }
    r.part = part;
    r.n_rows = n_rows;
    r.lim0 = ctx;
    r.s_off = 0;
    r.s_total = S;
    r.n_splits = S;
    const ProfRec pr = prof_rows(VC_PROF_VERIFY_ATTN, a, eb);
    vc_status st2 = launch_attn(a, d.dtype, s, pr.a, pr.b);
    if (st2) return st2;
    prof_commit(pr);
    CombineArgs c{};
    c.n_req = 1;
    c.n_rows = n_rows;
    c.Hq = d.n_q_heads;
    c.s_total = S;
    c.head_dim = d.head_dim;
    c.out_dtype = d.dtype;
    c.part[0] = part;
    c.out[0] = ob;
    c.s_used[0] = S;
    return launch_combine(c, s);
  };
  if ((st = forward_layers(m, n_rows, w8, L, tmpl, set_kv, attend, s))) return st;
  return head(m, 0, n_rows, w8, L, out_argmax, logits_opt, s);
}
}  // namespace

extern "C" {

vc_status vc_verify(vc_model* m, const vc_req* req, const void* staged_k, const void* staged_v, int32_t staged_cap,
                    const int32_t* tok, int32_t n_rows, int32_t* out_argmax, float* logits_opt, void* vtail_k,
                    void* vtail_v, int32_t vtail_cap, void* ws, size_t ws_bytes, hipStream_t s) {
  return verify_impl(m, req, staged_k, staged_v, staged_cap, tok, n_rows, out_argmax, logits_opt, vtail_k, vtail_v,
                     vtail_cap, ws, ws_bytes, nullptr, s);
}

vc_status vc_verify_layered(vc_model* m, const vc_req* req, const void* staged_k, const void* staged_v,
                            int32_t staged_cap, const int32_t* tok, int32_t n_rows, int32_t* out_argmax,
                            float* logits_opt, void* vtail_k, void* vtail_v, int32_t vtail_cap, void* ws,
                            size_t ws_bytes, const hipEvent_t* layer_ready, hipStream_t s) {
  VC_REQUIRE(layer_ready != nullptr, VC_ERR_ARG, "vc_verify_layered: null event array");
  return verify_impl(m, req, staged_k, staged_v, staged_cap, tok, n_rows, out_argmax, logits_opt, vtail_k, vtail_v,
                     vtail_cap, ws, ws_bytes, layer_ready, s);
}

vc_status vc_prefill(vc_model* m, const int32_t* tokens, int32_t T, void* k_out, void* v_out, int32_t cap, void* q_obs,
                     int32_t W, int32_t* g0_out, float* last_logits_opt, int32_t chunk, void* ws, size_t ws_bytes,
                     hipStream_t s) {
  if (vc_status st = check_model(m)) return st;
  VC_REQUIRE(tokens && k_out && v_out && g0_out && ws, VC_ERR_ARG, "vc_prefill: null argument");
  VC_REQUIRE(T > 0 && cap >= T && chunk > 0, VC_ERR_ARG, "vc_prefill: bad sizes");
  VC_REQUIRE(T <= m->d.max_pos, VC_ERR_CAPACITY, "vc_prefill: prompt beyond the RoPE table");
  VC_REQUIRE(q_obs == nullptr || (W > 0 && W <= T), VC_ERR_ARG, "vc_prefill: bad observation window");
  const vc_model_desc& d = m->d;
  const WsLayout L = ws_layout(m, chunk, T);
  VC_REQUIRE(ws_bytes >= L.total, VC_ERR_CAPACITY, "vc_prefill: workspace %zu < %zu bytes", ws_bytes, L.total);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  const int64_t Hkv = d.n_kv_heads, D = d.head_dim, eb = m->eb;
  const int64_t qrow = int64_t(d.n_q_heads) * D * eb;
  vc_status st;
  for (int c0 = 0; c0 < T; c0 += chunk) {
    const int C = std::min(chunk, T - c0);
    if ((st = k_embed(m->w.embed, tokens + c0, w8 + L.h, C, d.d_model, d.vocab, d.dtype, s))) return st;
    EpiArgs tmpl{};
    tmpl.batched = 0;
    tmpl.pos0 = c0;
    tmpl.row0 = c0;
    tmpl.pitch = cap;
    auto set_kv = [&](int l, EpiArgs& e) -> vc_status {
      e.kbase = mptr(k_out, l * Hkv * cap * D * eb);
      e.vbase = mptr(v_out, l * Hkv * cap * D * eb);
      return VC_OK;
    };
    auto attend = [&](int l, const void* qb, void* ob, float* part) -> vc_status {
      if (q_obs && c0 + C > T - W) {  // keep the observation queries of the last W prompt rows
        const int r_lo = std::max(c0, T - W);
        const int64_t bytes = int64_t(c0 + C - r_lo) * qrow;
        vc_status st3 = k_copy_words(cptr(qb, int64_t(r_lo - c0) * qrow),
                                     mptr(q_obs, (int64_t(l) * W + (r_lo - (T - W))) * qrow), bytes, s);
        if (st3) return st3;
      }
      AttnArgs a{};
      a.n_req = 1;
      a.Hq = d.n_q_heads;
      a.Hkv = d.n_kv_heads;
      a.G = d.n_q_heads / d.n_kv_heads;
      a.split_len = int(cdiv(c0 + C, ATT_KT) * ATT_KT);
      a.head_dim = d.head_dim;
      a.scale_log2 = LOG2E / sqrtf(float(D));
      a.n_rowblocks = int(cdiv(int64_t(C) * a.G, ATT_RB));
      a.max_splits = 1;
      AttnReq& r = a.r[0];
      r.q = qb;
      r.a = KVSeg{cptr(k_out, l * Hkv * cap * D * eb), cptr(v_out, l * Hkv * cap * D * eb), int64_t(cap) * D, c0 + C,
                  0};
      r.b = KVSeg{nullptr, nullptr, 0, 0, 0};
      r.part = part;
      r.n_rows = C;
      r.lim0 = c0;
      r.s_off = 0;
      r.s_total = 1;
      r.n_splits = 1;
      const ProfRec pr = prof_rows(VC_PROF_PREFILL_ATTN, a, eb);
      vc_status st2 = launch_attn(a, d.dtype, s, pr.a, pr.b);
      if (st2) return st2;
      prof_commit(pr);
      CombineArgs c{};
      c.n_req = 1;
      c.n_rows = C;
      c.Hq = d.n_q_heads;
      c.s_total = 1;
      c.head_dim = d.head_dim;
      c.out_dtype = d.dtype;
      c.part[0] = part;
      c.out[0] = ob;
      c.s_used[0] = 1;
      return launch_combine(c, s);
    };
    if ((st = forward_layers(m, C, w8, L, tmpl, set_kv, attend, s))) return st;
    if (c0 + C == T) {
      if ((st = head(m, C - 1, 1, w8, L, g0_out, last_logits_opt, s))) return st;
    }
  }
  return VC_OK;
}

vc_status vc_accept(vc_model* m, const vc_req* req, const int32_t* verified, int32_t x, const void* vtail_k,
                    const void* vtail_v, int32_t vtail_cap, int32_t* result, hipStream_t s) {
  if (vc_status st = check_model(m)) return st;
  VC_REQUIRE(req && req->rows && verified && vtail_k && vtail_v && result, VC_ERR_ARG, "vc_accept: null argument");
  VC_REQUIRE(x >= 0 && vtail_cap >= x + 1, VC_ERR_ARG, "vc_accept: bad draft length %d", x);
  VC_REQUIRE(req->tail_k && req->tail_v, VC_ERR_ARG, "vc_accept: request without tail");
  VC_REQUIRE(req->n_tail + x + 1 <= req->tail_cap, VC_ERR_CAPACITY, "vc_accept: tail capacity");
  const vc_model_desc& d = m->d;
  vc_status st;
  if ((st = k_accept(req->rows, verified, x, result, s))) return st;
  return k_commit_rows(vtail_k, vtail_v, vtail_cap, req->tail_k, req->tail_v, req->tail_cap, req->n_tail,
                       d.head_dim * m->eb, d.n_layers * d.n_kv_heads, x + 1, result, s);
}

vc_status vc_commit(vc_model* m, vc_req* req, int32_t a, const void* vtail_k, const void* vtail_v, int32_t vtail_cap,
                    hipEvent_t after, hipStream_t copy) {
  if (vc_status st = check_model(m)) return st;
  VC_REQUIRE(req && vtail_k && vtail_v, VC_ERR_ARG, "vc_commit: null argument");
  VC_REQUIRE(a >= 0 && a + 1 <= vtail_cap, VC_ERR_ARG, "vc_commit: bad accept count %d", a);
  const vc_model_desc& d = m->d;
  const size_t row = size_t(d.head_dim) * m->eb;
  if (req->comp != nullptr) {
    // VeriCache request: vc_accept already placed the verifier's rows in the device tail,
    // which is where the full cache keeps every committed row
    VC_REQUIRE(req->n_tail + a + 1 <= req->tail_cap, VC_ERR_CAPACITY, "vc_commit: tail capacity");
    req->ctx_len += a + 1;
    req->n_tail += a + 1;
    req->draft_idx = 0;
    return VC_OK;
  }
  VC_REQUIRE(req->ctx_len + a + 1 <= req->full_cap, VC_ERR_CAPACITY, "vc_commit: full KV capacity");
  if (after && !dbg_dry()) VC_HIP(hipStreamWaitEvent(copy, after, 0));
  if (req->full_k_host && req->full_v_host) {
    const size_t h = size_t(d.n_layers) * d.n_kv_heads;
    if (vc_status st = copy2d("commit K rows to the host", mptr(req->full_k_host, int64_t(req->ctx_len) * row),
                              size_t(req->full_cap) * row, vtail_k, size_t(vtail_cap) * row, size_t(a + 1) * row, h,
                              hipMemcpyDeviceToHost, copy))
      return st;
    if (vc_status st = copy2d("commit V rows to the host", mptr(req->full_v_host, int64_t(req->ctx_len) * row),
                              size_t(req->full_cap) * row, vtail_v, size_t(vtail_cap) * row, size_t(a + 1) * row, h,
                              hipMemcpyDeviceToHost, copy))
      return st;
  }
  req->ctx_len += a + 1;
  req->n_tail += a + 1;
  req->draft_idx = 0;
  return VC_OK;
}

vc_status vc_stage(vc_model* m, const vc_req* req, void* slot_k, void* slot_v, int32_t slot_cap, int32_t l0, int32_t l1,
                   hipStream_t copy) {
  if (vc_status st = check_model(m)) return st;
  VC_REQUIRE(req && slot_k && slot_v && req->full_k_host && req->full_v_host, VC_ERR_ARG, "vc_stage: null argument");
  const vc_model_desc& d = m->d;
  VC_REQUIRE(0 <= l0 && l0 <= l1 && l1 <= d.n_layers, VC_ERR_ARG, "vc_stage: bad layer range");
  HostPart hp;
  if (vc_status st = host_part(m, req, hp)) return st;
  const int rows = hp.rows;
  VC_REQUIRE(slot_cap >= rows && req->full_cap >= rows, VC_ERR_CAPACITY, "vc_stage: slot %d / host %d < %d rows",
             slot_cap, req->full_cap, rows);
  if (dbg_on()) {
    const int64_t lay = int64_t(d.n_kv_heads) * d.head_dim * m->eb * slot_cap;  // one layer of the slot
    if (vc_status st = dbg_request("vc_stage", m, *req, true, 1, l0, l1)) return st;
    if (vc_status st = dbg_check("vc_stage", {{"slot K", mptr(slot_k, l0 * lay), (l1 - l0) * lay},
                                              {"slot V", mptr(slot_v, l0 * lay), (l1 - l0) * lay}}))
      return st;
  }
  if (l0 == l1 || rows == 0) return VC_OK;
  const size_t row = size_t(d.head_dim) * m->eb;
  const int64_t lo_src = int64_t(l0) * d.n_kv_heads * req->full_cap * row;
  const int64_t lo_dst = int64_t(l0) * d.n_kv_heads * slot_cap * row;
  const size_t height = size_t(l1 - l0) * d.n_kv_heads;
  if (vc_status st = copy2d("stage K rows", mptr(slot_k, lo_dst), size_t(slot_cap) * row, cptr(req->full_k_host, lo_src),
                            size_t(req->full_cap) * row, size_t(rows) * row, height, hipMemcpyHostToDevice, copy))
    return st;
  return copy2d("stage V rows", mptr(slot_v, lo_dst), size_t(slot_cap) * row, cptr(req->full_v_host, lo_src),
                size_t(req->full_cap) * row, size_t(rows) * row, height, hipMemcpyHostToDevice, copy);
}

vc_status vc_host_alloc(size_t bytes, void** out_host) {
  VC_REQUIRE(out_host != nullptr && bytes > 0, VC_ERR_ARG, "vc_host_alloc: bad arguments");
  *out_host = nullptr;
  if (dbg_dry()) {
    *out_host = dbg_alloc(bytes, true);
    VC_REQUIRE(*out_host != nullptr, VC_ERR_HIP, "dry run: host allocation of %zu bytes failed", bytes);
    return VC_OK;
  }
  VC_HIP(hipHostMalloc(out_host, bytes, hipHostMallocDefault));
  dbg_register(*out_host, bytes);
  return VC_OK;
}

vc_status vc_host_free(void* host) {
  if (!host) return VC_OK;
  if (dbg_dry()) {
    dbg_free(host, true);
    return VC_OK;
  }
  dbg_forget(host);
  VC_HIP(hipHostFree(host));
  return VC_OK;
}

vc_status vc_offload(vc_model* m, const vc_req* req, const void* k_dev, const void* v_dev, int32_t src_cap, int32_t T,
                     hipStream_t s) {
  if (vc_status st = check_model(m)) return st;
  return vc_offload_layers(m, req, k_dev, v_dev, src_cap, T, 0, m->d.n_layers, s);
}

vc_status vc_offload_layers(vc_model* m, const vc_req* req, const void* k_dev, const void* v_dev, int32_t src_cap,
                            int32_t T, int32_t l0, int32_t l1, hipStream_t s) {
  if (vc_status st = check_model(m)) return st;
  VC_REQUIRE(req && k_dev && v_dev && req->full_k_host && req->full_v_host, VC_ERR_ARG, "vc_offload: null argument");
  VC_REQUIRE(T > 0 && T <= src_cap, VC_ERR_CAPACITY, "vc_offload: bad row counts");
  const vc_model_desc& d = m->d;
  VC_REQUIRE(0 <= l0 && l0 <= l1 && l1 <= d.n_layers, VC_ERR_ARG, "vc_offload: bad layer range");
  if (l0 == l1) return VC_OK;
  const size_t row = size_t(d.head_dim) * m->eb;
  const size_t height = size_t(l1 - l0) * d.n_kv_heads;
  if (req->comp != nullptr) {
    HostPart hp;
    vc_req probe = *req;
    probe.ctx_len = req->cd ? req->cd->seq_len + req->n_tail : 0;
    if (vc_status st = host_part(m, &probe, hp)) return st;
    VC_REQUIRE(T == hp.prompt, VC_ERR_ARG, "vc_offload: %d rows given for a %d-token prompt", T, hp.prompt);
    VC_REQUIRE(hp.rows <= req->full_cap, VC_ERR_CAPACITY, "vc_offload: host capacity %d < %d rows", req->full_cap,
               hp.rows);
    if (hp.split) {
      // the dropped rows, compacted, one layer at a time through a device staging buffer
      if (hp.rows == 0) return VC_OK;
      const size_t lbytes = size_t(d.n_kv_heads) * hp.rows * row;
      void* tmp = nullptr;
      if (vc_status st0 = dev_alloc(&tmp, 2 * lbytes)) return st0;
      vc_status st = VC_OK;
      for (int l = l0; l < l1 && st == VC_OK; l++) {
        for (int kv = 0; kv < 2 && st == VC_OK; kv++) {
          void* dst = mptr(tmp, kv * lbytes);
          st = gather_dropped(req->cd, req->comp, kv ? v_dev : k_dev, src_cap, l * d.n_kv_heads, d.n_kv_heads, dst,
                              hp.rows, s);
          if (st) break;
          void* host = kv ? req->full_v_host : req->full_k_host;
          st = copy2d("offload dropped rows", mptr(host, int64_t(l) * d.n_kv_heads * req->full_cap * row),
                      size_t(req->full_cap) * row, dst, size_t(hp.rows) * row, size_t(hp.rows) * row, d.n_kv_heads,
                      hipMemcpyDeviceToHost, s);
        }
      }
      const hipError_t e1 = dbg_dry() ? hipSuccess : hipStreamSynchronize(s);
      dev_free(tmp);
      if (st) return st;
      VC_HIP(e1);
      return VC_OK;
    }
  }
  VC_REQUIRE(T <= req->full_cap, VC_ERR_CAPACITY, "vc_offload: host capacity %d < %d rows", req->full_cap, T);
  const int64_t h0 = int64_t(l0) * d.n_kv_heads * req->full_cap * row, d0 = int64_t(l0) * d.n_kv_heads * src_cap * row;
  if (vc_status st = copy2d("offload K rows", mptr(req->full_k_host, h0), size_t(req->full_cap) * row, cptr(k_dev, d0),
                            size_t(src_cap) * row, size_t(T) * row, height, hipMemcpyDeviceToHost, s))
    return st;
  return copy2d("offload V rows", mptr(req->full_v_host, h0), size_t(req->full_cap) * row, cptr(v_dev, d0),
                size_t(src_cap) * row, size_t(T) * row, height, hipMemcpyDeviceToHost, s);
}

// ---------------------------------------------------------------- single-layer attention
vc_status vc_linear(const void* x, const void* w, float* y, int32_t M, int32_t N, int32_t K, int32_t dtype,
                    hipStream_t s) {
  VC_REQUIRE(x && w && y, VC_ERR_ARG, "vc_linear: null argument");
  VC_REQUIRE(M > 0 && N > 0 && K > 0, VC_ERR_ARG, "vc_linear: bad shape %d x %d x %d", M, N, K);
  VC_REQUIRE(dtype == VC_BF16 || dtype == VC_F32, VC_ERR_ARG, "vc_linear: bad dtype %d", dtype);
  return gemm(x, w, y, M, N, K, 1, dtype, s);
}

vc_status vc_attn_ws_size(const vc_attn_desc* d, int32_t n, int32_t rows, int32_t max_keys, size_t* bytes) {
  VC_REQUIRE(d && bytes && n > 0 && rows > 0 && max_keys > 0, VC_ERR_ARG, "vc_attn_ws_size: bad arguments");
  const int64_t D2 = d->head_dim + 2;
  VC_REQUIRE(d->n_kv_heads > 0 && d->n_q_heads % d->n_kv_heads == 0, VC_ERR_ARG, "vc_attn_ws_size: bad heads");
  const int sq = quant_split_len(d->n_q_heads / d->n_kv_heads, 64);  // quantized splits: shortest at group 64
  const int64_t S = cdiv(max_keys, SPLIT_DRAFT) + cdiv(max_keys, sq) + 2;
  *bytes = align256(size_t(n) * rows * d->n_q_heads * S * D2 * 4);
  return VC_OK;
}

vc_status vc_attn_draft(const vc_attn_desc* d, const vc_attn_draft_req* reqs, int32_t n, const void* q, void* out,
                        void* ws, size_t ws_bytes, hipStream_t s) {
  VC_REQUIRE(d && reqs && q && out && ws, VC_ERR_ARG, "vc_attn_draft: null argument");
  VC_REQUIRE(n > 0 && n <= VC_MAX_BATCH, VC_ERR_ARG, "vc_attn_draft: batch %d not in [1, %d]", n, VC_MAX_BATCH);
  VC_REQUIRE(d->n_kv_heads > 0 && d->n_q_heads % d->n_kv_heads == 0, VC_ERR_ARG, "vc_attn_draft: bad heads");
  CompView views[VC_MAX_BATCH];
  KVSeg tails[VC_MAX_BATCH];
  int tail_n[VC_MAX_BATCH];
  int max_keys = 1;
  for (int r = 0; r < n; r++) {
    if (vc_status st = comp_view(reqs[r].comp, reqs[r].cd, views[r])) return st;
    VC_REQUIRE(reqs[r].cd->n_layers == 1 && reqs[r].cd->n_kv_heads == d->n_kv_heads &&
                   reqs[r].cd->head_dim == d->head_dim && reqs[r].cd->dtype == d->dtype,
               VC_ERR_ARG, "vc_attn_draft: request %d has another shape", r);
    VC_REQUIRE(reqs[r].n_tail >= 0 && reqs[r].n_tail <= reqs[r].tail_cap, VC_ERR_ARG, "vc_attn_draft: bad tail");
    VC_REQUIRE(reqs[r].n_tail == 0 || (reqs[r].tail_k && reqs[r].tail_v), VC_ERR_ARG, "vc_attn_draft: null tail");
    tails[r] = KVSeg{reqs[r].tail_k, reqs[r].tail_v, int64_t(reqs[r].tail_cap) * d->head_dim, 0, 0};
    tail_n[r] = reqs[r].n_tail;
    max_keys = std::max(max_keys, views[r].lay.n_main + views[r].n_resid + tail_n[r]);
  }
  size_t need = 0;
  vc_attn_ws_size(d, n, 1, max_keys, &need);
  VC_REQUIRE(ws_bytes >= need, VC_ERR_CAPACITY, "vc_attn_draft: workspace %zu < %zu bytes", ws_bytes, need);
  VC_REQUIRE(d->out_dtype == VC_F32 || d->out_dtype == VC_BF16, VC_ERR_ARG, "vc_attn_draft: bad out_dtype");
  const int eb = d->dtype == VC_BF16 ? 2 : 4;
  const int ob = d->out_dtype == VC_BF16 ? 2 : 4;
  const int64_t stride = int64_t(d->n_q_heads) * d->head_dim * eb;
  const int64_t ostride = int64_t(d->n_q_heads) * d->head_dim * ob;
  return draft_attention(d->n_q_heads, d->n_kv_heads, d->head_dim, d->dtype, d->out_dtype, n, views, 0, tails, tail_n,
                         q, stride, out, ostride, static_cast<float*>(ws), s);
}

vc_status vc_attn_verify(const vc_attn_desc* d, int32_t n, const void* q, const void* const* staged_k,
                         const void* const* staged_v, int32_t staged_cap, const int32_t* ctx_host,
                         const void* const* tail_k, const void* const* tail_v, int32_t tail_cap, int32_t n_rows,
                         void* out, void* ws, size_t ws_bytes, hipStream_t s) {
  VC_REQUIRE(d && q && staged_k && staged_v && ctx_host && tail_k && tail_v && out && ws, VC_ERR_ARG,
             "vc_attn_verify: null argument");
  VC_REQUIRE(n > 0 && n <= VC_MAX_BATCH && n_rows > 0 && n_rows <= tail_cap, VC_ERR_ARG, "vc_attn_verify: bad sizes");
  VC_REQUIRE(d->n_kv_heads > 0 && d->n_q_heads % d->n_kv_heads == 0, VC_ERR_ARG, "vc_attn_verify: bad heads");
  VC_REQUIRE(d->out_dtype == VC_F32 || d->out_dtype == VC_BF16, VC_ERR_ARG, "vc_attn_verify: bad out_dtype");
  const int eb = d->dtype == VC_BF16 ? 2 : 4;
  const int ob = d->out_dtype == VC_BF16 ? 2 : 4;
  const int D = d->head_dim;
  const int split = d->split_len > 0 ? d->split_len : SPLIT_VERIFY;
  VC_REQUIRE(split % ATT_KT == 0, VC_ERR_ARG, "vc_attn_verify: split_len must be a multiple of 64");
  int max_keys = 1;
  for (int r = 0; r < n; r++) {
    VC_REQUIRE(ctx_host[r] >= 0 && ctx_host[r] <= staged_cap, VC_ERR_ARG, "vc_attn_verify: bad ctx");
    max_keys = std::max(max_keys, ctx_host[r] + n_rows);
  }
  const int S = int(cdiv(max_keys, split));
  const size_t need = align256(size_t(n) * n_rows * d->n_q_heads * S * (D + 2) * 4);
  VC_REQUIRE(ws_bytes >= need, VC_ERR_CAPACITY, "vc_attn_verify: workspace %zu < %zu bytes", ws_bytes, need);
  float* part = static_cast<float*>(ws);
  const int64_t per_req = int64_t(n_rows) * d->n_q_heads * S * (D + 2);
  const int64_t qstride = int64_t(n_rows) * d->n_q_heads * D * eb;
  AttnArgs a{};
  a.n_req = n;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.G = d->n_q_heads / d->n_kv_heads;
  a.split_len = split;
  a.head_dim = D;
  a.scale_log2 = LOG2E / sqrtf(float(D));
  a.n_rowblocks = int(cdiv(int64_t(n_rows) * a.G, ATT_RB));
  a.max_splits = S;
  CombineArgs c{};
  c.n_req = n;
  c.n_rows = n_rows;
  c.Hq = d->n_q_heads;
  c.s_total = S;
  c.head_dim = D;
  c.out_dtype = d->out_dtype;
  const int64_t ostride = int64_t(n_rows) * d->n_q_heads * D * ob;
  for (int r = 0; r < n; r++) {
    AttnReq& ar = a.r[r];
    ar.q = cptr(q, r * qstride);
    ar.a = KVSeg{staged_k[r], staged_v[r], int64_t(staged_cap) * D, ctx_host[r], 0};
    ar.b = KVSeg{tail_k[r], tail_v[r], int64_t(tail_cap) * D, n_rows, 0};
    ar.part = part + r * per_req;
    ar.n_rows = n_rows;
    ar.lim0 = ctx_host[r];
    ar.s_off = 0;
    ar.s_total = S;
    ar.n_splits = int(cdiv(ctx_host[r] + n_rows, split));
    c.part[r] = ar.part;
    c.out[r] = mptr(out, r * ostride);
    c.s_used[r] = ar.n_splits;
  }
  const ProfRec pr = prof_rows(VC_PROF_VERIFY_ATTN, a, eb);
  vc_status st = launch_attn(a, d->dtype, s, pr.a, pr.b);
  if (st) return st;
  prof_commit(pr);
  return launch_combine(c, s);
}

}  // extern "C"
