/*
 * vc.h -- C ABI of the VeriCache draft/verify hot path for AMD MI355X (gfx950).
 *
 * Method (cited by page title and section):
 *   "VeriCache: Making Lossy KV Compression Exact" (devshah.ca), "The Core Idea":
 *     the same weights draft x tokens greedily over a compressed KV cache; one
 *     verification forward over the full KV cache returns x + 1 predictions
 *     (one per drafted position plus a bonus); tokens are accepted left to right
 *     until the first mismatch, where the full-cache token is emitted instead;
 *     when every draft matches the bonus token is emitted too.
 *   Same page, "Verifying Without Giving Back the Speedup": the full cache lives
 *     off the GPU and is brought in only to verify; verification is staggered
 *     across requests so transfers overlap other requests' drafting.
 *   "VeriCache Guide: Lossless Inference with Lossy KV Caches" (aifetchly),
 *     "The Uniform Compressor Interface": compress(full_k, full_v) -> (ck, cv)
 *     for token-eviction and low-bit quantization families.
 *
 * Conventions
 *   Pointers are device pointers unless the name ends in _host (pinned host
 *   memory from hipHostMalloc).  Every buffer is allocated and owned by the
 *   caller; the library allocates nothing on the hot path (vc_model_create
 *   allocates its RoPE table once and vc_model_destroy frees it).
 *   Element types: VC_F32 (IEEE float) or VC_BF16 (bfloat16 bit patterns).
 *   KV rows are head-major: a cache buffer of one request is
 *   [L][Hkv][cap][D], row t of (layer l, head j) at ((l*Hkv + j)*cap + t)*D.
 *   All entry points only enqueue work on the given stream(s) and return;
 *   kernel faults surface at the caller's next synchronisation.  Calls are
 *   thread-compatible, not thread-safe: do not share one vc_model between
 *   threads without external locking.
 *   Outputs are bitwise reproducible, and the arithmetic of each verify row
 *   does not depend on how many rows are verified together nor on whether a
 *   key sits in the staged cache or in the verify tail (row invariance), so
 *   vc_verify with n_rows = 1 is full-KV greedy decoding with exactly the
 *   tokens VeriCache emits.
 *   Token ids: every argmax the library writes (drafts, verified tokens, g0) is
 *   the lowest index of the largest logit, or -1 when the row's logits have no
 *   finite maximum (all NaN, or all -inf).  An input token outside [0, vocab)
 *   (such a -1 included) reads no memory: its embedding row is quiet NaN, so
 *   that row's outputs are NaN and its argmax is -1 again (NaN keys or values
 *   reach every row that shares their 64-key attention tile, the rows before
 *   them included: the masked weights are zero and 0 x NaN is NaN).  A caller
 *   that sees -1 has non-finite activations upstream and should stop decoding
 *   that request.
 *
 * Errors: every call returns vc_status; 0 is success.  Negative values:
 *   VC_ERR_ARG (null pointer, bad shape or size), VC_ERR_UNSUPPORTED (e.g. a
 *   head_dim or bit width the kernels do not implement), VC_ERR_CAPACITY (a
 *   workspace, tail or slot too small), VC_ERR_HIP (a HIP launch or copy
 *   failed).  vc_last_error() returns a message for the calling thread.
 */
#ifndef VC_H
#define VC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vc_status;
#define VC_OK 0
#define VC_ERR_ARG (-1)
#define VC_ERR_UNSUPPORTED (-2)
#define VC_ERR_CAPACITY (-3)
#define VC_ERR_HIP (-4)

#define VC_F32 0
#define VC_BF16 1

#define VC_TOKDROP 1
#define VC_QUANT 2
/* token-drop ranking (vc_compress_desc.score) */
#define VC_SCORE_ATTN 0    /* observed attention of the last obs_window prompt queries */
#define VC_SCORE_KEYNORM 1 /* key norm ("The Uniform Compressor Interface" example)     */

#define VC_MAX_BATCH 16 /* requests per vc_draft_step / vc_attn_* call */

const char* vc_last_error(void);
int32_t vc_abi_version(void);

/* ------------------------------------------------------------------------
 * Model: a pre-norm decoder (RMSNorm, rotate-half RoPE, GQA attention,
 * SwiGLU FFN, untied LM head).  The pages do not describe the architecture;
 * this is the Llama-style reading of the workloads' shapes.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t dtype;    /* VC_F32 (head_dim 64) or VC_BF16 (head_dim 128) */
  float rope_theta; /* RoPE base */
  float eps;        /* RMSNorm epsilon */
  int32_t max_pos;  /* highest position + 1 the RoPE table must cover */
} vc_model_desc;

/* Weight pointers (caller-owned, model dtype, matrices row-major [out][in]). */
typedef struct {
  const void* embed;      /* [V][d]                                            */
  const void* lm_head;    /* [V][d]                                            */
  const void* norm_final; /* [d]                                               */
  const void* norm_attn;  /* [L][d]                                            */
  const void* norm_ffn;   /* [L][d]                                            */
  const void* w_qkv;      /* [L][(Hq + 2 Hkv) D][d]: rows of Wq, then Wk, then Wv */
  const void* w_o;        /* [L][d][Hq D] (Hq D need not equal d)              */
  const void* w_gu;       /* [L][2 ffn][d]: rows of W1 (gate), then W3 (up)    */
  const void* w_down;     /* [L][d][ffn]                                       */
} vc_weights;

typedef struct vc_model vc_model;

/* Validates shapes, copies the descriptor and pointers, and builds the RoPE
 * cos/sin table (angles in float64, stored float32).  For bf16 models it also
 * keeps a copy of w_qkv, w_o, w_gu, w_down and lm_head in a fragment-major
 * layout (1 KB tiles of 16 rows x 32 columns in the order the weight-streaming
 * GEMMs of draft steps and verification read them; as much device memory as
 * those weights), so those weights must hold their final values when the model
 * is created; prefill reads the caller's row-major weights.  Synchronises `s`. */
vc_status vc_model_create(const vc_model_desc* desc, const vc_weights* w, hipStream_t s, vc_model** out);
vc_status vc_model_destroy(vc_model* m);

/* Workspace bytes for vc_draft_step / vc_verify / vc_prefill with at most
 * max_rows rows per call (draft batch, x + 1, or prefill chunk) and at most
 * max_keys keys visible to any row. */
vc_status vc_ws_size(const vc_model* m, int32_t max_rows, int32_t max_keys, size_t* bytes);

/* ------------------------------------------------------------------------
 * Compression ("The Uniform Compressor Interface").  Input: one request's
 * full K (after RoPE) and V, [L][Hkv][src_cap][D] in `dtype`, rows [0, seq_len).
 *
 * VC_TOKDROP: per (layer, KV head), score each candidate row t < T - R by the
 *   mean over the GQA group's observation queries of its causal softmax
 *   probability (q_obs [L][W][Hq][D] in dtype: the post-RoPE queries of the
 *   last W prompt positions); keep the top keep_total - R candidates (ties to
 *   the smaller index) plus the last R rows, ascending.  Output blob:
 *     K_keep [L][Hkv][Kk][D] dtype | V_keep same | idx [L][Hkv][Kk] int32 |
 *     keep_mask [L][Hkv][nt] u64 | keep_cnt [L][Hkv][nt] int32
 *   with Kk = min(T, max(keep_total, min(R, T))) and nt = ceil(T/64): bit o of
 *   keep_mask[tile] says whether position 64*tile + o is kept, keep_cnt[tile]
 *   counts the kept positions before the tile.  A position t is then K_keep row
 *   cnt + (kept below it in the tile) when kept, else dropped row
 *   t - cnt - (kept below it): the compacted order in which the host holds the
 *   dropped rows (vc_offload) and verification stages them.
 *   score = VC_SCORE_KEYNORM ranks by key norm instead ([VC2] "The Uniform
 *   Compressor Interface", its example compressor): per layer, e[t] = mean over
 *   the KV heads of ||k_t||_2 in float32 (channels summed in order, heads in
 *   order), one ranking shared by every head of the layer; the top
 *   keep_total - R rows by e (ties to the smaller index) plus the last R rows
 *   (R = keep_recent, 0 for the pages' rule), same blob; q_obs is not read and
 *   obs_window is ignored.
 * VC_QUANT: b in {2,3,4} bits, group G in {64,128}, Tq = floor(T/G)*G.
 *   K per channel (groups of G tokens), V per token (groups of G channels):
 *   zero = fp16(min), scale = fp16((max - min) / (2^b - 1)),
 *   code = scale == 0 ? 0 : clamp(rint((x - zero) / scale), 0, 2^b - 1),
 *   IEEE float32 arithmetic.  Output blob:
 *     Kc [L][Hkv][Tq][D*b/8]        u8  token rows; channel d at bits [d*b, d*b+b)
 *     Vc [L][Hkv][Tq/64][D][64*b/8] u8  per channel, 64 tokens; token i at bits [i*b, i*b+b)
 *     Ks, Kz [L][Hkv][Tq/G][D]      fp16
 *     Vs, Vz [L][Hkv][Tq][D/G]      fp16
 *     Kr, Vr [L][Hkv][T-Tq][D]      dtype (rows left unquantized)
 *   Bitstreams are little-endian (stream bit n = bit n%8 of byte n/8).
 * Every section starts at a multiple of 256 bytes.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t kind;                                /* VC_TOKDROP | VC_QUANT            */
  int32_t bits, group;                         /* VC_QUANT                         */
  int32_t keep_total, keep_recent, obs_window; /* VC_TOKDROP                       */
  int32_t n_layers, n_q_heads, n_kv_heads, head_dim, seq_len, dtype;
  int32_t src_cap; /* row pitch (rows) of the input K/V per (layer, head) */
  int32_t score;   /* VC_TOKDROP ranking: VC_SCORE_ATTN | VC_SCORE_KEYNORM */
} vc_compress_desc;

/* Byte offsets of the sections of a compressed blob. */
typedef struct {
  size_t total;
  int32_t n_main;  /* Kk (token drop) or Tq (quant): rows in the main region     */
  int32_t n_resid; /* rows left unquantized (quant); 0 for token drop            */
  size_t k_main, v_main, idx;       /* token drop: K_keep, V_keep, idx           */
  size_t kc, vc, ks, kz, vs, vz;    /* quant                                     */
  size_t kr, vr;                    /* quant residual rows                       */
  size_t keep_mask, keep_cnt;       /* token drop: per-tile kept map (below)      */
  int32_t n_tiles;                  /* token drop: ceil(T / 64)                   */
  int32_t n_host;  /* prompt rows per (layer, head) that only the host holds:
                      T - Kk (token drop: the dropped rows), T (quant)              */
} vc_compress_layout;

vc_status vc_compress_layout_of(const vc_compress_desc* d, vc_compress_layout* out);
vc_status vc_compress_size(const vc_compress_desc* d, size_t* out_bytes, size_t* ws_bytes);
vc_status vc_compress(const vc_compress_desc* d, const void* k, const void* v, const void* q_obs, void* out,
                      size_t out_bytes, void* ws, size_t ws_bytes, hipStream_t s);

/* ------------------------------------------------------------------------
 * Per-request state (host struct, caller-owned).
 *   tail: exact rows after the compressed region (and after the quantizer's
 *         residual rows, which stay in the blob), [L][Hkv][tail_cap][D] in
 *         the model dtype: the verifier's rows of every committed token;
 *         during a round the draft rows follow at n_tail + draft_idx.
 *   ctx_len: rows in the full KV = absolute position of the pending token
 *         (prompt length T + n_tail for a request with a compressed cache).
 *   The full KV of a request with a compressed cache is split by where its
 *   exact rows already are: the device holds the committed rows (tail) and,
 *   for token drop, the kept prompt rows; the pinned host buffer holds the
 *   other n_host prompt rows per (layer, head) (vc_compress_layout.n_host:
 *   the dropped rows compacted in position order, or all T rows for quant),
 *   and only those cross PCIe for a verification.  A request with comp ==
 *   NULL is plain: the host holds its whole context (full-KV decoding).
 * ---------------------------------------------------------------------- */
typedef struct {
  const void* comp;          /* compressed blob (device)                                */
  const vc_compress_desc* cd;
  void* tail_k;
  void* tail_v;
  int32_t tail_cap, n_tail;
  int32_t ctx_len;
  int32_t draft_idx;         /* step within the current round (vc_draft_step)           */
  void* full_k_host;         /* pinned [L][Hkv][full_cap][D]: host rows (see above)     */
  void* full_v_host;
  int32_t full_cap;
  int32_t* rows;             /* device int32 [>= x + 1]: rows[0] = pending token,        */
                             /* rows[1 + i] = draft i of the current round              */
} vc_req;

/* One batched greedy draft step over the compressed caches ("The Core Idea":
 * the compressed-cache model autoregressively produces the draft).  Request r
 * consumes rows[draft_idx] at position ctx_len + draft_idx, writes its K/V row to
 * tail row n_tail + draft_idx, attends over the compressed region (including a
 * quantizer's residual rows) and tail rows [0, n_tail + draft_idx], and writes
 * rows[draft_idx + 1] = argmax (ties to the lowest id).  The caller advances
 * draft_idx.  logits_opt: device float [n][V] or NULL. */
vc_status vc_draft_step(vc_model* m, const vc_req* reqs, int32_t n, float* logits_opt, void* ws, size_t ws_bytes,
                        hipStream_t s);

/* vc_draft_step for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same step, with its
 * workspace in a library-owned static device array of VC_STATIC_SCRATCH_BYTES per GPU (each
 * GPU that runs the library holds its own copy until the process ends) instead of a caller
 * buffer; its outputs equal vc_draft_step's bit for bit.  Returns VC_ERR_CAPACITY when the step
 * needs more workspace than that (vc_ws_size(m, n, max keys visible to a request) bytes;
 * 16 requests of the 8B-shaped model at 131072 keys need about 120 MiB).  Every call on one
 * GPU uses that GPU's one array, which keeps the previous call's contents (the step writes
 * every byte it reads): calls that overlap on one GPU, from several streams or threads, race.
 * Allocates nothing. */
#define VC_STATIC_SCRATCH_BYTES (160u << 20)
#define VC_MAX_DEVICES 64
vc_status vc_draft_step_static(vc_model* m, const vc_req* reqs, int32_t n, float* logits_opt, hipStream_t s);

/* Verification forward of ONE request ("The Core Idea": predictions for every
 * drafted position plus one bonus, in a single pass against the full cache).
 * Rows tok[0..n_rows) (the pending token then the x drafts) sit at positions
 * ctx_len .. ctx_len + n_rows - 1; row i attends to the full KV of positions
 * [0, ctx_len) and verify rows 0..i, keys taken in position order from the
 * staged host rows, the kept rows of a token-drop cache and the tail (see the
 * per-request state).  Writes out_argmax[n_rows] and the exact K/V of every row
 * into vtail [L][Hkv][vtail_cap][D].  staged_k/v: [L][Hkv][staged_cap][D] in
 * the model dtype holding the request's host rows (vc_stage).  Each key
 * contributes the same arithmetic whichever buffer holds it, so a request with
 * a compressed cache verifies bit for bit like a plain request over the same
 * full KV.  n_rows = 1 is greedy decoding. */
vc_status vc_verify(vc_model* m, const vc_req* req, const void* staged_k, const void* staged_v, int32_t staged_cap,
                    const int32_t* tok, int32_t n_rows, int32_t* out_argmax, float* logits_opt, void* vtail_k,
                    void* vtail_v, int32_t vtail_cap, void* ws, size_t ws_bytes, hipStream_t s);

/* vc_verify with the staged rows arriving layer by layer (the swap cost of
 * bringing the full KV back, "The VeriCache Architecture", VeriCache Guide):
 * layer_ready holds n_layers events (host array of handles); before layer l's
 * attention reads the staged rows, `s` waits for layer_ready[l], which the
 * caller records on its copy stream once layer l is staged (vc_stage with
 * l0 = l, l1 = l + 1).  Each layer's projections run before that wait, and
 * layer l's compute overlaps the copies of the later layers.  Results are
 * those of vc_verify.  The events are not retained after the call returns
 * (the waits are enqueued). */
vc_status vc_verify_layered(vc_model* m, const vc_req* req, const void* staged_k, const void* staged_v,
                            int32_t staged_cap, const int32_t* tok, int32_t n_rows, int32_t* out_argmax,
                            float* logits_opt, void* vtail_k, void* vtail_v, int32_t vtail_cap, void* ws,
                            size_t ws_bytes, const hipEvent_t* layer_ready, hipStream_t s);

/* Accept until the first mismatch ("The Core Idea", pseudocode and worked
 * example).  On `s`: with draft = req->rows + 1, a = first i < x with
 * draft[i] != verified[i] (else x); result[0] = a, result[1 .. a+1] =
 * draft[0..a) followed by verified[a] (the correction, or the bonus token when
 * a == x); req->rows[0] = verified[a] (the next pending token); then the
 * verifier's rows 0..a are copied from vtail into the request's tail at n_tail
 * (overwriting this round's draft rows).  verified: device int32 [x+1];
 * result: device int32 [x+2].  x = 0 is a plain round (no drafts: the pending
 * token alone was verified, and its successor is emitted).  Does not block and does not change *req:
 * after result[0] is visible on the host, call vc_commit.
 * This splits the single accept-and-commit call of the four-call interface
 * sketched for the method: accepting runs on the device and returns no host
 * count, and the host copy of the accepted rows (for a plain request only;
 * a compressed request keeps them exact in its device tail) moves to
 * vc_commit, so nothing here waits on the host. */
vc_status vc_accept(vc_model* m, const vc_req* req, const int32_t* verified, int32_t x, const void* vtail_k,
                    const void* vtail_v, int32_t vtail_cap, int32_t* result, hipStream_t s);

/* Host half of the commit, after result[0] = a is known: advance req->n_tail
 * and req->ctx_len by a + 1 and reset draft_idx.  A request with a compressed
 * cache keeps its committed rows in the device tail (vc_accept wrote them), so
 * nothing is copied.  A plain request gets vtail rows 0..a appended to its
 * pinned full KV at row ctx_len, enqueued on `copy` after `after` (may be
 * NULL). */
vc_status vc_commit(vc_model* m, vc_req* req, int32_t a, const void* vtail_k, const void* vtail_v, int32_t vtail_cap,
                    hipEvent_t after, hipStream_t copy);

/* Pinned host memory of exactly `bytes` bytes (hipHostMalloc) for a full KV
 * cache, and its release.  Setup-time helpers, not for the hot path. */
vc_status vc_host_alloc(size_t bytes, void** out_host);
vc_status vc_host_free(void* host);

/* Offload (setup): from a device cache [L][Hkv][src_cap][D] holding prompt rows
 * [0, T), copy the request's host rows into its pinned buffer on `s`: the
 * dropped rows, compacted, for token drop (through a temporary device buffer;
 * the call then synchronises `s`), all T rows otherwise. */
vc_status vc_offload(vc_model* m, const vc_req* req, const void* k_dev, const void* v_dev, int32_t src_cap, int32_t T,
                     hipStream_t s);
/* vc_offload of layers [l0, l1) only.  Like vc_stage, it touches only those
 * layers of the host arrays (bytes [l0, l1) x Hkv x full_cap x D x elem of
 * full_k_host / full_v_host), so a caller that keeps host rows in ordinary
 * (pageable) memory can move them one layer at a time through a pinned buffer
 * of one layer, passing full_k_host = buffer - l0 x (that layer size): the
 * library never hands pageable memory to a copy engine. */
vc_status vc_offload_layers(vc_model* m, const vc_req* req, const void* k_dev, const void* v_dev, int32_t src_cap,
                            int32_t T, int32_t l0, int32_t l1, hipStream_t s);

/* Stage the request's host rows (n_host per (layer, head) with a compressed
 * cache, ctx_len for a plain request) from pinned host memory into a device
 * slot [L][Hkv][slot_cap][D] on `copy` (SDMA, hipMemcpy2DAsync), layers
 * [l0, l1); only those layers of the host arrays and the slot are touched. */
vc_status vc_stage(vc_model* m, const vc_req* req, void* slot_k, void* slot_v, int32_t slot_cap, int32_t l0, int32_t l1,
                   hipStream_t copy);

/* Prefill of one prompt (untimed setup): tokens[0..T) at positions 0..T-1 in
 * chunks of `chunk` rows, each through the verification path with the rows
 * before it as the staged cache.  Writes K/V into k_out/v_out
 * [L][Hkv][cap][D], the post-RoPE queries of the last W rows into q_obs
 * [L][W][Hq][D] (NULL to skip), g0 = argmax of row T-1 into g0_out[0], and
 * row T-1's logits into last_logits_opt [V] (NULL to skip; sampled decoding
 * draws g0 from them with vc_sample). */
vc_status vc_prefill(vc_model* m, const int32_t* tokens, int32_t T, void* k_out, void* v_out, int32_t cap,
                     void* q_obs, int32_t W, int32_t* g0_out, float* last_logits_opt, int32_t chunk, void* ws,
                     size_t ws_bytes, hipStream_t s);

/* One projection of the model's linear layers (every GEMM of prefill, draft
 * and verification; the model itself is the pre-norm decoder of the
 * configurations, since the pages fix no architecture), in a single K range:
 * y[M][N] (float32) = x[M][K] w[N][K]^T, the products of dtype elements summed
 * in float32.  M > 64 runs the prefill kernel (256 x 256 MFMA tiles when N is a
 * multiple of 256, else 128 x 128), M <= 64 the weight-streaming kernel of the
 * decode steps.  dtype VC_BF16 needs K % 128 == 0 and N % 64 == 0 (M <= 64) or
 * N % 128 == 0 (M > 64); VC_F32 takes any shape.  Row-major device buffers,
 * caller-owned; y is overwritten.  VC_ERR_ARG for a non-positive size, a null
 * pointer or another dtype, VC_ERR_UNSUPPORTED for a shape outside the above. */
vc_status vc_linear(const void* x, const void* w, float* y, int32_t M, int32_t N, int32_t K, int32_t dtype,
                    hipStream_t s);

/* ------------------------------------------------------------------------
 * Sampled decoding ("VeriCache Guide: Lossless Inference with Lossy KV
 * Caches", "Mathematical Guarantee of Lossless Correctness"): drafts are drawn
 * from the compressed-cache distribution, and a draft x is kept with
 * probability min(1, p_target(x) / p_draft(x)), where p_target is the full-KV
 * verification row's distribution; at the first rejection the token is drawn
 * from max(0, p_target - p_draft) renormalised, and after x kept drafts the
 * bonus token from verify row x.  Every emitted token is then distributed as
 * full-KV sampling would draw it.
 *   Distribution of a logits row: softmax(logits / temperature); temperature 0
 *   is the one-hot row at the greedy argmax (the whole path then emits the
 *   greedy tokens).  A row holding NaN or +inf, or nothing finite, draws -1.
 *   Draws: inverse CDF, the lowest index i of positive weight whose running
 *   sum (a fixed-order fp32 scan) exceeds u * (total).  u comes from
 *   Philox4x64-10 (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2,
 *   3", SC 2011) with key (seed, 0) and counter (position, purpose, stream, 0):
 *   (first output word >> 40) * 2^-24.  position is the absolute position of
 *   the token being chosen; purpose is one of VC_DRAW_*.
 * ---------------------------------------------------------------------- */
typedef struct {
  float temperature; /* finite, >= 0 */
  uint64_t seed;     /* generator key word 0                        */
  uint64_t stream;   /* counter word 2: one stream per request      */
} vc_sampler;
#define VC_DRAW_DRAFT 0  /* a draft token                                       */
#define VC_DRAW_ACCEPT 1 /* the acceptance test of a draft                      */
#define VC_DRAW_TARGET 2 /* a token drawn from the target: g0, plain sampling, the
                            token after a rejection, the bonus token            */

/* One token per logits row: row r (logits + r * vocab, device fp32) with
 * sampler smp[r] (host array) at position pos[r] (host array) and draw
 * `purpose`; writes out_tok[r] (device) and, when probs_opt is not NULL, the
 * row's distribution to probs_opt + r * vocab (device fp32). */
vc_status vc_sample(const float* logits, int32_t n_rows, int32_t vocab, const vc_sampler* smp, const int64_t* pos,
                    int32_t purpose, int32_t* out_tok, float* probs_opt, hipStream_t s);

/* vc_draft_step with the draft token drawn instead of the argmax: request r
 * draws rows[draft_idx + 1] at position ctx_len + draft_idx + 1 with smp[r]
 * (VC_DRAW_DRAFT) and writes the draft distribution to probs[r] + draft_idx *
 * vocab (probs: host array of n device pointers, each to [>= x][vocab] fp32,
 * which vc_spec_sample reads after the round's x steps). */
vc_status vc_draft_step_sampled(vc_model* m, const vc_req* reqs, int32_t n, const vc_sampler* smp,
                                float* const* probs, float* logits_opt, void* ws, size_t ws_bytes, hipStream_t s);

/* Speculative rejection sampling of one verified round of one request: the
 * step that replaces the greedy comparison before vc_accept.  logits_t: the
 * x + 1 verify rows' logits (vc_verify's logits_opt, device fp32
 * [x + 1][vocab]); probs_d: the draft distributions [x][vocab] (from
 * vc_draft_step_sampled); draft: the x drafts (req->rows + 1); pos0: the
 * pending token's position (req->ctx_len), so draft i sits at pos0 + 1 + i.
 * Draft i is kept when u_accept * p_d(draft i) < p_t(draft i); with a the
 * first rejection (else x), writes verified[0..a) = the kept drafts and
 * verified[a] = the token drawn with the TARGET draw of its position from the
 * residual of row a (from row x when a = x; from row a without the rejected
 * draft if rounding left the residual no mass), which always differs from a
 * rejected draft, so that vc_accept then finds the same a and emits it.
 * verified[i > a] is not written.  ws: device, vc_spec_ws_size bytes. */
vc_status vc_spec_ws_size(int32_t x, size_t* bytes);
vc_status vc_spec_sample(int32_t vocab, const float* logits_t, const float* probs_d, const int32_t* draft, int32_t x,
                         const vc_sampler* smp, int64_t pos0, int32_t* verified, void* ws, size_t ws_bytes,
                         hipStream_t s);

/* ------------------------------------------------------------------------
 * Attention cores of one layer (the single-layer workload and tests).
 * Query rows are [rows][Hq][D] bf16 (post-RoPE); outputs [rows][Hq][D] in out_dtype.
 *
 * Value range.  Draft attention over a bf16 token-drop cache keeps V in bf16
 * (P.V on bf16 MFMAs with P as a bf16 hi/lo pair): any finite bf16 V.
 * Verification (and prefill) attention runs P.V on fp16 MFMAs, so each bf16 V
 * element is converted to fp16 there: the contract is |v| <= 65504, and it
 * binds every model call, since each one verifies or prefills.  Inside it the
 * conversion is exact for |v| >= 2^-14 and off by at most 2^-25 (absolute)
 * below.  An element beyond it becomes +-inf and makes the output channels it
 * feeds non-finite (never a finite wrong value); through a model this reaches
 * the logits, and the argmax then writes -1 (see the token-id conventions).
 * The quantized compressor stores fp16 scales and zeros, so the same bound
 * holds for the range max - min of every quantization group.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t n_q_heads, n_kv_heads, head_dim, dtype;
  int32_t split_len; /* keys per split-K partial, multiple of 64 (0 = library default) */
  int32_t out_dtype; /* VC_F32 or VC_BF16 element type of `out` (bf16 = round to nearest even of the fp32 result) */
} vc_attn_desc;

typedef struct {
  const void* comp;            /* compressed blob of ONE layer (L = 1 in its descriptor) */
  const vc_compress_desc* cd;
  const void* tail_k;          /* [Hkv][tail_cap][D] */
  const void* tail_v;
  int32_t tail_cap;
  int32_t n_tail;              /* tail rows visible to the draft row (own row included) */
} vc_attn_draft_req;

/* Decode attention of one query row per request over its compressed main
 * region (dequantized in registers, or the kept rows) followed by its tail
 * rows, split-K partials merged in ascending split order. q: [n][Hq][D]. */
vc_status vc_attn_draft(const vc_attn_desc* d, const vc_attn_draft_req* reqs, int32_t n, const void* q, void* out,
                        void* ws, size_t ws_bytes, hipStream_t s);

/* Verification attention of n_rows rows per request: row i of request r sees
 * staged rows [0, ctx) and tail rows 0..i.  Arrays have n entries. q:
 * [n][n_rows][Hq][D]; staged_k/v: per request [Hkv][staged_cap][D];
 * tail_k/v: per request [Hkv][tail_cap][D]; out like q. */
vc_status vc_attn_verify(const vc_attn_desc* d, int32_t n, const void* q, const void* const* staged_k,
                         const void* const* staged_v, int32_t staged_cap, const int32_t* ctx_host,
                         const void* const* tail_k, const void* const* tail_v, int32_t tail_cap, int32_t n_rows,
                         void* out, void* ws, size_t ws_bytes, hipStream_t s);

vc_status vc_attn_ws_size(const vc_attn_desc* d, int32_t n, int32_t rows, int32_t max_keys, size_t* bytes);

/* ------------------------------------------------------------------------
 * Live measurement of kernel classes, for benchmarks.  When the class's bit
 * (1 << kind) is enabled, every launch of that class records a HIP event pair
 * taken at the kernel's own start and end on its stream, together with the
 * algorithmic bytes the launch must move and the flops it must compute:
 *   VC_PROF_DRAFT_ATTN    draft-step attention partials of all requests of one
 *                         layer (one pair spans the quantized and the exact-row
 *                         launch): compressed main region (codes, scales and zeros,
 *                         or kept rows), exact tail rows, queries (split partials
 *                         in aux_bytes);
 *   VC_PROF_VERIFY_ATTN   verification attention of one layer: every key visible to
 *                         the last row, K and V once per KV head, queries (partials
 *                         in aux_bytes); flops 4 D Hq per (row, visible key);
 *   VC_PROF_GEMM_SKINNY   projection / LM-head GEMM with M <= 64 rows (weights and X;
 *                         float32 partials in aux_bytes; flops 2 M N K);
 *   VC_PROF_GEMM_TILED    the same for larger M (prefill chunks);
 *   VC_PROF_PREFILL_ATTN  causal prefill attention of one chunk (bytes as for
 *                         verification; its keys are read once per row group).
 * vc_profile_read synchronises the recorded events of one class, returns the
 * totals and clears that class's record.  Not thread-safe.
 * ---------------------------------------------------------------------- */
#define VC_PROF_DRAFT_ATTN 0
#define VC_PROF_VERIFY_ATTN 1
#define VC_PROF_GEMM_SKINNY 2
#define VC_PROF_GEMM_TILED 3
#define VC_PROF_PREFILL_ATTN 4
#define VC_PROF_KINDS 5
typedef struct {
  int64_t launches;   /* timed launches (or launch groups)                  */
  double total_ms;    /* summed event time of those launches               */
  double bytes;       /* summed algorithmic bytes                          */
  double flops;       /* summed algorithmic flops                          */
  double aux_bytes;   /* bytes beyond the algorithmic ones: the launches'
                         own split-K partials (written, and read back by
                         the combine or the epilogue)                      */
} vc_profile_stats;
/* mask: bit k enables class k (0 disables all). */
vc_status vc_profile_enable(uint32_t mask);
vc_status vc_profile_read(int32_t kind, vc_profile_stats* out);

/* ------------------------------------------------------------------------
 * Address-range checking (debugging, not for the hot path).
 *   VC_DEBUG_CHECK: before every kernel launch and copy the library states
 *     each byte range it will touch, from the call's arguments and the
 *     kernel's own loop bounds, and checks that each lies inside one buffer
 *     registered with vc_debug_register (device or host memory; the library
 *     registers what it allocates itself: the RoPE table, pinned buffers of
 *     vc_host_alloc, temporaries, the static scratch).  A range outside every
 *     buffer fails the call with VC_ERR_ARG before anything is launched;
 *     vc_last_error() names the kernel, the operand and the range.
 *   VC_DEBUG_DRY: the same checks, and then no HIP call at all (no launch,
 *     copy, event, synchronisation or device allocation; vc_host_alloc and
 *     the library's temporaries become lazily mapped host memory, and
 *     host_alloc bytes are counted as pinned).  A caller passes host memory
 *     where device buffers would be, and replays a workload's exact sequence
 *     of calls on a machine without a GPU.  Results are not computed: device
 *     outputs keep whatever the caller's buffers held.
 *   Not thread-safe with respect to mode changes.
 * ---------------------------------------------------------------------- */
#define VC_DEBUG_OFF 0
#define VC_DEBUG_CHECK 1
#define VC_DEBUG_DRY 2
typedef struct {
  int64_t launches;    /* launches and copies checked            */
  int64_t ranges;      /* byte ranges checked                    */
  int64_t violations;  /* checks that failed                     */
  double pinned_bytes; /* vc_host_alloc bytes live (dry mode)    */
  double pinned_peak;  /* their peak                             */
} vc_debug_stats;
vc_status vc_debug_mode(int32_t mode);
vc_status vc_debug_register(const void* p, size_t bytes);
vc_status vc_debug_forget(const void* p);
/* Counters since the last reset; reset != 0 clears them (the live pinned bytes are kept). */
vc_status vc_debug_stats_read(vc_debug_stats* out, int32_t reset);

/* ------------------------------------------------------------------------
 * Seeded synthetic inputs (not part of the method): the counter-based
 * SplitMix64 generator of the input recipe, evaluated on the GPU so that
 * large workloads need not be generated on the host.  Counter
 * c = stream*2^40 + seed*2^32 + index, u = (splitmix64(c) >> 40) * 2^-24.
 * ---------------------------------------------------------------------- */
/* dst[i] = round((2u(start+i) - 1) * sqrt(6/(fan_in+fan_out))), i < n, dtype VC_F32 or VC_BF16
 * (float64 -> float32 -> bf16, each round-to-nearest-even). */
vc_status vc_synth_xavier(void* dst, int32_t dtype, int64_t n, uint32_t stream, uint32_t seed, int64_t start,
                          int32_t fan_in, int32_t fan_out, hipStream_t s);
/* Box-Muller normals into bf16 [B][H][rows][D] (element index = counter index),
 * columns outl[(b*H+h)*n_outl + k] of head (b, h) multiplied by outl_scale
 * before rounding; outl may be NULL. */
vc_status vc_synth_normal_heads(void* dst_bf16, int32_t B, int32_t H, int32_t rows, int32_t D, uint32_t stream,
                                uint32_t seed, const int32_t* outl, int32_t n_outl, float outl_scale, hipStream_t s);
vc_status vc_synth_ids(int32_t* dst, int64_t n, uint32_t stream, uint32_t seed, int32_t vocab, hipStream_t s);
vc_status vc_synth_fill(void* dst, int32_t dtype, int64_t n, float value, hipStream_t s);

#ifdef __cplusplus
}
#endif
#endif /* VC_H */
