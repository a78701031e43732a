/*
 * kvp.h - C ABI of libkvp: learned KV-cache eviction and GQA decode attention over
 * the pruned, paged cache, for AMD Instinct MI355X (gfx950).
 *
 * Method sources (page title and section; see the repository's design notes for
 * the readings taken where the pages are silent):
 *   KVzap  - "NVIDIA open-sources KVzap" digest (max5.ai), key points: a surrogate
 *            model predicts an importance score per cache entry from hidden states;
 *            a single linear layer or a 2-layer MLP; low scores are removed while the
 *            most recent 128 tokens are always kept.
 *   DMS    - "Nvidia's new technique cuts LLM reasoning cost 8x" (euno.news), "How
 *            DMS works" (binary keep/evict signal per token) and "Delayed Eviction"
 *            (a flagged token stays for a short window, then leaves the cache).
 *   BeaconKV - paper briefing (jiinsi.com), body: important tokens at full
 *            precision, the rest lossily compressed (low-precision quantization).
 *   DeInfer - gist.science summary of arXiv 2604.17709, method part (b): a remapping
 *            index list and a compact, fixed-address KV buffer make the decode step
 *            capturable in a static graph.
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller (structs themselves
 *     live in host memory).  The library allocates nothing, keeps no hidden state
 *     between calls (one exception: the fixed per-GPU scratch behind
 *     kvp_decode_attn_noalloc), and never synchronises, except kvp_check().
 *   - Every call enqueues its kernels on `stream` and returns at once; outputs are
 *     valid once the stream reaches that point.  Calls on different streams must use
 *     disjoint buffers.
 *   - Argument errors are found on the host before anything is enqueued and return
 *     KVP_E_ARG / KVP_E_DTYPE / KVP_E_WORKSPACE / KVP_E_UNSUPPORTED.  A failed
 *     launch returns KVP_E_HIP.  Pool overflow found on the device sets bits in
 *     kv->err, which kvp_check() reports as KVP_E_CAPACITY.  No C++ exception
 *     crosses this boundary.
 *   - bf16 is passed as raw 16-bit patterns; scores and outputs are fp32.
 */
#ifndef KVP_H
#define KVP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVP_PAGE 16 /* tokens per page */

typedef enum kvp_status {
  KVP_OK = 0,
  KVP_E_ARG = 1,         /* null pointer, bad shape, inconsistent sizes */
  KVP_E_DTYPE = 2,       /* dtype combination not supported */
  KVP_E_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace_size() */
  KVP_E_CAPACITY = 4,    /* a page pool or block table ran out (device-detected) */
  KVP_E_HIP = 5,         /* a HIP runtime call or kernel launch failed */
  KVP_E_UNSUPPORTED = 6  /* valid request the library does not implement */
} kvp_status;

typedef enum kvp_dtype { KVP_F32 = 0, KVP_BF16 = 1 } kvp_dtype;

/* Device error bits accumulated in kvp_paged_kv.err (sticky until kvp_clear_error). */
#define KVP_ERR_POOL_FULL 0x1   /* main page pool exhausted */
#define KVP_ERR_TABLE_FULL 0x2  /* a pair needs more pages than max_pages_per_pair */
#define KVP_ERR_POOL8_FULL 0x4  /* int8 pool or its block table exhausted */

/* kvp_paged_kv.lp_bits: code format of the low-precision pool. */
#define KVP_LP_INT8 8          /* int8 codes (0 means the same) */
#define KVP_LP_INT4 4          /* int4 codes, two per byte */
#define KVP_LP_FP8_E4M3 0x108  /* OCP FP8 E4M3 codes, one per byte (8-bit code width in the
                                  low byte, bit 8 marks floating-point codes) */

/* ----------------------------------------------------------------------------
 * Surrogate scorer weights (KVzap, key points: surrogate model / structure).
 * nn.Linear layout [out][in].
 *   LINEAR: s = x W^T + b1            w1 [Hkv][H] (dtype wdtype), b1 [Hkv] or NULL
 *   MLP:    s = GELU(x W1^T + b1) W2^T + b2   (exact erf GELU)
 *           w1 [inner][H] (wdtype), b1 [inner] or NULL, w2 [Hkv][inner] fp32,
 *           b2 [Hkv] or NULL.
 * wdtype must equal the hidden-state dtype.  MLP requires bf16, H % 64 == 0,
 * inner % 256 == 0 and Hkv <= 16; LINEAR requires Hkv <= 16 (and H % 32 == 0 for
 * bf16).  Both need a workspace for some shapes (see kvp_score_workspace_size):
 * the MLP for its per-slice partial scores, and either kind for small batches
 * (<= 64 tokens, H % 256 == 0, H <= 8192), which split the contraction over K.
 * -------------------------------------------------------------------------- */
typedef enum kvp_scorer_kind { KVP_SCORER_LINEAR = 0, KVP_SCORER_MLP = 1 } kvp_scorer_kind;

typedef struct kvp_scorer {
  int32_t kind;       /* kvp_scorer_kind */
  int32_t hidden;     /* H */
  int32_t inner;      /* MLP width (ignored for LINEAR) */
  int32_t n_kv_heads; /* Hkv: one score per KV head */
  int32_t wdtype;     /* kvp_dtype of w1 */
  int32_t _pad;
  const void* w1;
  const float* b1;
  const float* w2;
  const float* b2;
} kvp_scorer;

/* ----------------------------------------------------------------------------
 * Paged KV cache, one block table per (batch, KV head) "pair" since keep masks
 * differ per head.  Page p of the main pool holds up to 16 tokens of one pair:
 *   k_pages [num_pages][16][d]   token-major K page
 *   v_pages [num_pages][d][16]   dim-major V page (V^T of the page)
 *   page_pos [num_pages][16]     absolute position of each slot
 * block_table[pair][j] is the physical page of the pair's j-th page; the pair holds
 * length[pair] tokens in its pages, in ascending position order.  page_top[0] is a
 * bump allocator over the pool.  The optional low-precision pool (BeaconKV
 * demotion; all fields NULL/0 when absent) has the same layout with codes plus one
 * fp32 absmax scale per slot for K and for V: lp_bits = KVP_LP_INT8 holds int8 codes
 * (-127..127, scale = absmax/127), KVP_LP_INT4 int4 codes (-7..7, scale = absmax/7)
 * two per byte, the even element in the low nibble (K rows: dims 2i, 2i+1; V^T rows:
 * tokens 2i, 2i+1), so its pages are half the size, and KVP_LP_FP8_E4M3 OCP FP8 E4M3
 * codes one per byte (scale = absmax/448; code = E4M3 rounding, to nearest even, of
 * the fp32 quotient value/scale).  Source: BeaconKV briefing (jiinsi.com), body and
 * FAQ: non-beacon entries are kept at low precision; the format is not given there.
 * Physical page ids and the unused slots of partly filled pages are unspecified.
 * -------------------------------------------------------------------------- */
typedef struct kvp_paged_kv {
  int32_t dtype;              /* KVP_BF16 or KVP_F32 (main pool element type) */
  int32_t num_pairs;          /* B * Hkv */
  int32_t head_dim;           /* d: 64 or 128 */
  int32_t num_pages;          /* main pool capacity in pages */
  int32_t max_pages_per_pair; /* row stride of block_table */
  int32_t num_pages8;         /* low-precision pool capacity (0 = no such pool) */
  int32_t max_pages8_per_pair;
  int32_t lp_bits;            /* code format of that pool: KVP_LP_INT8 (or 0), KVP_LP_INT4,
                                 KVP_LP_FP8_E4M3 */
  void* k_pages;
  void* v_pages;
  int32_t* page_pos;
  int32_t* block_table; /* [num_pairs][max_pages_per_pair] */
  int32_t* length;      /* [num_pairs] */
  int32_t* page_top;    /* [1] */
  int32_t* err;         /* [1] KVP_ERR_* bits */
  int8_t* k8_pages;     /* [num_pages8][16][d] code bytes ([16][d/2] for int4) */
  int8_t* v8_pages;     /* [num_pages8][d][16] code bytes ([d][8] for int4) */
  float* k8_scale;      /* [num_pages8][16] */
  float* v8_scale;      /* [num_pages8][16] */
  int32_t* page8_pos;   /* [num_pages8][16] */
  int32_t* block_table8; /* [num_pairs][max_pages8_per_pair] */
  int32_t* length8;     /* [num_pairs] */
  int32_t* page8_top;   /* [1] */
} kvp_paged_kv;

/* ----------------------------------------------------------------------------
 * Recent-window ring (the always-kept recent tokens / the DMS delay buffer).
 * Position t of a pair lives in slot t mod window while it is among the last
 * `window` positions.  Storage per pair is window/16 pages in the main-pool
 * layout: k [num_pairs][window/16][16][d], v [num_pairs][window/16][d][16];
 * score [num_pairs][window] is the slot's score, pos [num_pairs][window] its
 * absolute position or -1 when empty.  Element type = kv->dtype.
 * window must be a positive multiple of 16, at most 1024.
 * -------------------------------------------------------------------------- */
typedef struct kvp_ring {
  int32_t window;
  int32_t _pad;
  void* k;
  void* v;
  float* score;
  int32_t* pos;
} kvp_ring;

typedef enum kvp_compact_mode {
  KVP_COMPACT_EVICT = 0,      /* evicted tokens are dropped */
  KVP_COMPACT_DEMOTE_INT8 = 1 /* evicted tokens go to the low-precision pool (BeaconKV;
                                 int8 or int4 codes per kv->lp_bits) */
} kvp_compact_mode;

/* Human-readable name of a status code (static string, never NULL). */
const char* kvp_status_str(kvp_status s);

/* Library version string. */
const char* kvp_version(void);

/* ----------------------------------------------------------------------------
 * kvp_score - surrogate importance score per (token, KV head).
 * Source: KVzap, key points (surrogate model over hidden states; linear or
 * 2-layer MLP structure; practical application: one score per cache entry).
 *   hidden  [B][T][H] contiguous, dtype hdtype (== sc->wdtype)
 *   scores  [B][Hkv][ld_s] fp32 (ld_s >= T); element (b,h,t) at (b*Hkv+h)*ld_s+t
 *   ws      workspace of at least kvp_score_workspace_size(sc, B, T) bytes (may be
 *           NULL when that size is 0)
 * Errors: KVP_E_ARG (null/shape), KVP_E_DTYPE, KVP_E_UNSUPPORTED, KVP_E_WORKSPACE.
 * -------------------------------------------------------------------------- */
kvp_status kvp_score(const kvp_scorer* sc, const void* hidden, int32_t hdtype, int32_t B,
                     int32_t T, float* scores, int64_t ld_s, void* ws, size_t ws_bytes,
                     hipStream_t stream);
size_t kvp_score_workspace_size(const kvp_scorer* sc, int32_t B, int32_t T);

/* ----------------------------------------------------------------------------
 * kvp_select - keep mask, per-pair kept count and ordered index lists.
 * Source: KVzap, key points, practical application (low scores removed, the most
 * recent 128 tokens always kept).
 *   keep[p][t] = (scores[p][t] >= tau) || (t >= T - recent); NaN scores fail the
 *   comparison.  p = b*Hkv + h.
 *   keep_bits  [B*Hkv][ceil(T/32)] u32, bit t%32 of word t/32 (tail bits zero)
 *   kept_idx   [B*Hkv][T] i32: the kept positions ascending in [0, count), then the
 *              evicted positions ascending in [count, T)
 *   kept_count [B*Hkv] i32
 *   ws         >= kvp_select_workspace_size(B, Hkv, T) bytes
 * T >= 1, recent >= 0.
 * -------------------------------------------------------------------------- */
kvp_status kvp_select(const float* scores, int32_t B, int32_t Hkv, int32_t T, int64_t ld_s,
                      float tau, int32_t recent, uint32_t* keep_bits, int32_t* kept_idx,
                      int32_t* kept_count, void* ws, size_t ws_bytes, hipStream_t stream);
size_t kvp_select_workspace_size(int32_t B, int32_t Hkv, int32_t T);

/* kvp_select_dev_tau - kvp_select with tau read from device memory (tau[0]), e.g.
 * as written by kvp_threshold, so the prefill needs no host round trip.  Same
 * arguments, rules and errors as kvp_select; tau == NULL is KVP_E_ARG. */
kvp_status kvp_select_dev_tau(const float* scores, int32_t B, int32_t Hkv, int32_t T,
                              int64_t ld_s, const float* tau, int32_t recent, uint32_t* keep_bits,
                              int32_t* kept_idx, int32_t* kept_count, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* ----------------------------------------------------------------------------
 * kvp_threshold - on-device threshold for a keep ratio.
 * Source: KVzap, key points (entries scoring below a threshold are removed):
 * keeping a fraction k of the entries is thresholding at the (1 - k) quantile.
 *   tau_out[0] (device memory) = fp32 rounding of the q-quantile of the N = B*Hkv*T
 *   scores (the first T of each row of [B*Hkv][ld_s]) by numpy's default "linear"
 *   rule: sorted ascending a[0..N-1], v = (N - 1) q, a[floor v] moved towards
 *   a[floor v + 1] by v - floor v (a[N-1] when v >= N - 1), interpolated in fp64.
 *   Any NaN score gives NaN.  q in [0, 1] (else KVP_E_ARG); N < 2^32 and
 *   B*Hkv <= 65535 (else KVP_E_UNSUPPORTED).  Exact (radix select, not sampling).
 *   ws >= kvp_threshold_workspace_size() bytes (scratch, any contents).
 * -------------------------------------------------------------------------- */
kvp_status kvp_threshold(const float* scores, int32_t B, int32_t Hkv, int32_t T, int64_t ld_s,
                         double q, float* tau_out, void* ws, size_t ws_bytes, hipStream_t stream);
size_t kvp_threshold_workspace_size(void);

/* ----------------------------------------------------------------------------
 * kvp_compact - rebuild the paged cache from a dense context and a selection.
 * Source: DeInfer method (b) (a remapping index list drives a copy into a compact,
 * fixed-address cache); KVzap practical application (only kept entries remain);
 * BeaconKV body (DEMOTE_INT8: non-beacon entries stored at low precision).
 *   k, v       dense [B][Hkv][T][d], dtype == kv->dtype, d == kv->head_dim
 *   kept_idx, kept_count  as written by kvp_select for the same (B, Hkv, T)
 *   scores     [B][Hkv][ld_s]; read only when ring != NULL (ring slot scores)
 *   ring       optional.  With a ring, kept positions t >= T - window go to ring
 *              slot t mod window (the other slots are emptied) and only older kept
 *              positions go to the pool; without one, every kept position goes to
 *              the pool.
 *   mode       EVICT drops non-kept positions.  DEMOTE_INT8 quantizes them into the
 *              int8 pool (symmetric absmax per (token, head), separately for K and
 *              V, fp32 scale = absmax/127, round-half-even, clamp to +-127).
 * The main (and int8) pool are reset: page_top, lengths and block tables are
 * rewritten; pages are handed out pair by pair.  Overflow sets kv->err bits and the
 * affected pairs keep what fits.  ws >= kvp_compact_workspace_size(B, Hkv).
 * -------------------------------------------------------------------------- */
kvp_status kvp_compact(const void* k, const void* v, int32_t dtype, int32_t B, int32_t Hkv,
                       int32_t T, int32_t d, const int32_t* kept_idx,
                       const int32_t* kept_count, const float* scores, int64_t ld_s,
                       int32_t mode, const kvp_paged_kv* kv, const kvp_ring* ring, void* ws,
                       size_t ws_bytes, hipStream_t stream);
size_t kvp_compact_workspace_size(int32_t B, int32_t Hkv);

/* ----------------------------------------------------------------------------
 * kvp_step_delayed - one decode step of the recent-window ring with delayed
 * eviction.  Source: DMS "Delayed Eviction" (a flagged token stays for a fixed
 * window of steps, then is removed); KVzap practical application (recent tokens
 * always kept, low scores removed).
 * For every pair: the token at position p - window leaves ring slot p mod window
 * and is appended to the pool iff its score >= tau (else dropped, or demoted to the
 * int8 pool when kv has one); then the new token (k_new, v_new, s_new) enters the
 * slot with position p.  With tau = 0 and window = w this is DMS; with
 * window = recent it continues KVzap's rule during decode.
 *   k_new, v_new [B*Hkv][d] dtype == kv->dtype;  s_new: score of pair i at
 *   s_new[i * ld_s]; p >= 0 is the absolute position of the new token (the same
 *   for every pair).  Pages are allocated from page_top; overflow sets kv->err.
 * -------------------------------------------------------------------------- */
kvp_status kvp_step_delayed(const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                            const void* v_new, int32_t dtype, const float* s_new,
                            int64_t ld_s, float tau, int32_t p, hipStream_t stream);

/* kvp_step_delayed_dev - kvp_step_delayed with every per-step value in device memory,
 * so the call can sit in a captured HIP graph and be replayed step after step (the
 * fixed-address decode step of the DeInfer methodology, part (b)).
 *   tau  device float: tau[0] (e.g. written by kvp_threshold)
 *   pos  device int32[2]: pos[0] = absolute position of the new token; pos[1] must be 0
 *        (arrival count).  On completion pos[0] has advanced by 1 and pos[1] is 0 again.
 * tau == NULL or pos == NULL is KVP_E_ARG; otherwise as kvp_step_delayed. */
kvp_status kvp_step_delayed_dev(const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                                const void* v_new, int32_t dtype, const float* s_new,
                                int64_t ld_s, const float* tau, int32_t* pos, hipStream_t stream);

/* kvp_score_step_delayed - kvp_step_delayed_dev with the new tokens' scores computed by
 * the scorer inside the step.  Sources: KVzap key points (a single linear layer or a
 * two-layer MLP over the hidden states as the surrogate scorer); DMS "Delayed Eviction"
 * (the step); DeInfer methodology (b) (a fixed-address decode step replayed from a graph).
 *   sc          n_kv_heads = Hkv with num_pairs = B * Hkv (Hkv <= 16)
 *               LINEAR: w1 [Hkv][H], b1 [Hkv] or NULL; one kernel.  hidden_new and w1
 *                 16-byte aligned and H a multiple of 8 (bf16) or 4 (fp32), else
 *                 KVP_E_ARG / KVP_E_UNSUPPORTED.  Score = x . w1[h] + b1[h] summed in
 *                 fp32 (bf16 products are exact).
 *               MLP: bf16, B <= 64, H a multiple of 256 and <= 8192, inner a multiple
 *                 of 256 and <= 1024 (else KVP_E_UNSUPPORTED); two kernels: the split-K
 *                 partial sums of the first layer (as kvp_score for small batches), then
 *                 the step, whose wave per pair adds the slices, b1, GELU, W2 row h and
 *                 b2.  ws >= kvp_score_workspace_size(sc, B, 1) bytes, 16-byte aligned,
 *                 as are b1 and w2 (KVP_E_WORKSPACE / KVP_E_ARG).
 *               Either score may differ from kvp_score's value for the same token in the
 *               last bits (another summation order).
 *   hidden_new  [B][H] hidden states of the new tokens, hdtype == sc->wdtype
 *   s_new       NULL, or [B * Hkv] fp32 output: the scores the ring stores for the new
 *               tokens, pair i = b * Hkv + h at s_new[i]
 *   tau, pos    device values exactly as in kvp_step_delayed_dev (both required)
 *   ws          MLP only (may be NULL for LINEAR)
 * Everything else is kvp_step_delayed_dev with s_new = that score. */
kvp_status kvp_score_step_delayed(const kvp_scorer* sc, const void* hidden_new, int32_t hdtype,
                                  const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                                  const void* v_new, int32_t dtype, float* s_new, const float* tau,
                                  int32_t* pos, void* ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------------------------------
 * kvp_decode_attn - GQA decode attention over the kept entries only.
 * Source: KVzap key points (GQA does not shorten the sequence axis; pruning does);
 * BeaconKV body (full-precision and low-precision entries read together).
 *   q   [B][Hq][d], dtype qdtype == kv->dtype; query head j reads KV head j / g,
 *       g = Hq / Hkv (contiguous head groups), g <= 16
 *   out [B][Hq][d] fp32: softmax(sm_scale * K q) V over the pair's pool tokens, its
 *       non-empty ring slots and (if present) its int8 tokens, all in one softmax.
 *       A pair with no visible token yields zeros.
 *   ws  >= kvp_decode_attn_workspace_size(...) bytes of scratch (any contents),
 *       256-byte aligned; it holds the page prefix of the split and the partial
 *       (max, sum, output) records between the two kernels.
 * Work split: the kept pages of all pairs form one sequence (and the low-precision
 * pages another), cut into one contiguous share per wave; each share is walked 32
 * tokens at a time and leaves one partial record per pair it touches; a second kernel
 * merges each pair's records in page order, so the output does not depend on timing
 * (bit-identical reruns).  The split's page prefix lives in each work-group's LDS up to
 * ~20000 pairs (~10000 with a low-precision pool); beyond that a third kernel (one
 * work-group) writes it to the workspace first and the waves read it from there (slower
 * per pair boundary, same results).
 * -------------------------------------------------------------------------- */
kvp_status kvp_decode_attn(const void* q, int32_t qdtype, int32_t B, int32_t Hq,
                           const kvp_paged_kv* kv, const kvp_ring* ring, float sm_scale,
                           float* out, void* ws, size_t ws_bytes, hipStream_t stream);
size_t kvp_decode_attn_workspace_size(int32_t B, int32_t Hq, int32_t num_pairs,
                                      int32_t head_dim);

/* ----------------------------------------------------------------------------
 * kvp_decode_step - one whole decode step in one call: the delayed step (with the new
 * tokens scored by the surrogate scorer, or scores given) followed by the decode
 * attention over the cache it leaves.  Sources: DMS "Delayed Eviction" (the step);
 * KVzap key points (surrogate scorer; attention over the kept entries only); DeInfer
 * methodology (b) (a fixed-address decode step replayed from a graph).
 * Equivalent to kvp_score_step_delayed (sc != NULL) or kvp_step_delayed_dev (sc == NULL,
 * scores s_in[pair * ld_s]) followed by kvp_decode_attn with the same q: the cache, the
 * device position, the stored scores and s_out are bit-identical to that sequence's; out
 * agrees to fp32 rounding (the tokens are summed in another grouping).  The work runs in
 * the attention's two kernels: the streaming kernel reads the cache as the step will
 * leave it (the token leaving its ring slot counts iff it is retained; the new token is
 * read from k_new/v_new) without writing it, and with an MLP scorer also computes the
 * split-K partial sums of the new tokens' first layer; the merge kernel finishes the
 * scores and applies the step.  The call launches kernels only and takes tau and the
 * position from device memory, so it can be captured in a HIP graph and replayed: one step
 * per graph, or several consecutive steps in one graph (the position advances on the
 * device from one to the next; each captured step reads its inputs at the addresses it
 * was captured with), which pays the runtime's per-replay start-up once for all of them.
 *   sc, hidden_new, hdtype  as kvp_score_step_delayed (sc->n_kv_heads = num_pairs / B), or
 *                sc == NULL: hidden_new unused, scores from s_in (ld_s >= 1)
 *   k_new, v_new [B*Hkv][d] bf16, 16-byte aligned; s_out NULL or [B*Hkv] fp32 (scorer)
 *   tau, pos     device values as in kvp_step_delayed_dev (tau[0]; pos[0] the position
 *                appended, advanced by 1; pos[1] must be 0 and is left 0)
 *   q, qdtype, B, Hq, sm_scale, out  as kvp_decode_attn
 *   ws           >= kvp_decode_step_workspace_size(sc, B, Hq, num_pairs, head_dim) bytes,
 *                256-byte aligned, scratch (any contents)
 * Takes bf16 caches with a ring and no low-precision pool (else KVP_E_UNSUPPORTED: make
 * the separate calls).  If the pool or a block table overflows (kv->err, kvp_check), this
 * step's output may include the retained token the pool could not take.
 * -------------------------------------------------------------------------- */
kvp_status kvp_decode_step(const kvp_scorer* sc, const void* hidden_new, int32_t hdtype,
                           const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                           const void* v_new, const float* s_in, int64_t ld_s, float* s_out,
                           const float* tau, int32_t* pos, const void* q, int32_t qdtype,
                           int32_t B, int32_t Hq, float sm_scale, float* out, void* ws,
                           size_t ws_bytes, hipStream_t stream);
size_t kvp_decode_step_workspace_size(const kvp_scorer* sc, int32_t B, int32_t Hq,
                                      int32_t num_pairs, int32_t head_dim);

/* ----------------------------------------------------------------------------
 * kvp_decode_attn_noalloc -kvp_decode_attn for callers that cannot allocate device
 * memory at all (code under HIP graph capture, tight serving loops, hosts that forbid
 * hipMalloc): no workspace argument; the library's own fixed device scratch of
 * KVP_NOALLOC_SCRATCH_BYTES, one copy per GPU, reserved when the library's code is
 * loaded on that GPU and held until the process ends, takes its place.  The call
 * itself allocates nothing (no hipMalloc, no hipFree).
 *   Arguments, layouts, output and errors as kvp_decode_attn, and the same kernels, so
 *   the output is bit-identical to kvp_decode_attn's.  Additionally:
 *   KVP_E_WORKSPACE  kvp_decode_attn_workspace_size(B, Hq, num_pairs, head_dim) exceeds
 *                    KVP_NOALLOC_SCRATCH_BYTES (g = 4, d = 128 fits up to 14043 pairs,
 *                    g = 8 up to 6009, g = 16 up to 1983)
 *   KVP_E_ARG        `stream` belongs to another device than the current one
 * The scratch is shared by every call on one GPU and keeps the last call's contents
 * (nothing in it needs to start at zero): calls that overlap in time on one GPU, on
 * different streams or from different threads, race and give undefined outputs.
 * Serialise them (one stream, or events).
 * -------------------------------------------------------------------------- */
#define KVP_NOALLOC_SCRATCH_BYTES (64u << 20) /* 64 MiB per GPU */
kvp_status kvp_decode_attn_noalloc(const void* q, int32_t qdtype, int32_t B, int32_t Hq,
                                   const kvp_paged_kv* kv, const kvp_ring* ring, float sm_scale,
                                   float* out, hipStream_t stream);

/* ----------------------------------------------------------------------------
 * kvp_prefill_attn - causal attention of every prompt position over the keys the
 * cache still holds for it.
 * Source: DMS "Delayed Eviction" (a flagged token stays readable for a window of
 * steps, then leaves); KVzap key points (low-scoring entries removed, recent ones
 * kept).  Position i of the prompt sees key j iff j <= i and (keep bit j is set or
 * i - j < window): what the decode step at length i + 1 sees.  KVzap: the selection
 * of kvp_select(tau, recent) with window = recent; DMS: kvp_select(0, w) with
 * window = w.
 *   q          [B][Hq][T][d] bf16; query head j reads KV head j / g, g = Hq / Hkv
 *   k, v       [B][Hkv][T][d] bf16 (dtype must be KVP_BF16), finite
 *   keep_bits  [B*Hkv][ceil(T/32)] u32, bit t%32 of word t/32 (tail bits ignored)
 *   kept_idx   [B*Hkv][T] i32 whose first (number of set bits) entries are the kept
 *              positions ascending -- as written by kvp_select for the same keep bits
 *   out        [B][Hq][T][d] fp32: softmax(sm_scale * K q_i) V over the keys position
 *              i sees; a row that sees no key (window 0, nothing kept before it) is 0
 * g in {1, 2, 4, 8, 16} and d in {64, 128} (else KVP_E_UNSUPPORTED); T >= 1, window >= 0,
 * sm_scale finite and > 0 (else KVP_E_ARG).
 * All buffers are caller-owned device memory; no workspace, no allocation.
 * -------------------------------------------------------------------------- */
kvp_status kvp_prefill_attn(const void* q, const void* k, const void* v, int32_t dtype,
                            int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d,
                            const uint32_t* keep_bits, const int32_t* kept_idx,
                            int32_t window, float sm_scale, float* out, hipStream_t stream);

/* ----------------------------------------------------------------------------
 * Helpers.
 * kvp_reset: empty the pools (lengths 0, page_top 0) and, if ring != NULL, the
 *            ring (pos -1).  Stream-ordered, no allocation.
 * kvp_clear_error: zero kv->err.
 * kvp_check: synchronise `stream`, read kv->err; KVP_E_CAPACITY if any bit is set.
 * -------------------------------------------------------------------------- */
kvp_status kvp_reset(const kvp_paged_kv* kv, const kvp_ring* ring, hipStream_t stream);
kvp_status kvp_clear_error(const kvp_paged_kv* kv, hipStream_t stream);
kvp_status kvp_check(const kvp_paged_kv* kv, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVP_H */
