// extern "C" entry points of libkvp: argument validation on the host, then the
// stream-ordered kernel launches in the per-step translation units.  Nothing here
// allocates or synchronises (except kvp_check), and no exception escapes.
#include <string.h>

#include <mutex>

#include "kvp_internal.h"

// launchers (defined next to their kernels)
kvp_status kvp_launch_score(const kvp_scorer* sc, const void* hidden, int B, int T, float* scores,
                            int64_t ld_s, void* ws, hipStream_t stream);
kvp_status kvp_launch_select(const float* scores, int num_pairs, int T, int64_t ld_s, float tau,
                             const float* tau_dev, int recent, uint32_t* bits, int* kept_idx,
                             int* kept_count, void* ws, hipStream_t stream);
kvp_status kvp_launch_threshold(const float* scores, int rows, int T, int64_t ld_s, double q,
                                float* tau_out, void* ws, hipStream_t stream);
kvp_status kvp_launch_compact(const void* k, const void* v, int num_pairs, int T, int d,
                              const int* kept_idx, const int* kept_count, const float* scores,
                              int64_t ld_s, int demote, const kvp_paged_kv* kv, const kvp_ring* ring,
                              void* ws, hipStream_t stream);
kvp_status kvp_launch_step_delayed(const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                                   const void* v_new, const float* s_new, int64_t ld_s, float tau,
                                   const float* tau_dev, int p, int* pos_dev, hipStream_t stream,
                                   const kvp_scorer* sc = nullptr, const void* x_new = nullptr,
                                   float* s_out = nullptr, const float* part = nullptr);
bool kvp_score_small_mlp_ok(const kvp_scorer* sc, int ntok);
kvp_status kvp_launch_score_small_partials(const kvp_scorer* sc, const void* hidden, int ntok,
                                           float* part, hipStream_t stream);
kvp_status kvp_launch_decode_attn(const void* q, int B, int Hq, const kvp_paged_kv* kv,
                                  const kvp_ring* ring, float sm_scale, float* out, void* ws,
                                  size_t ws_bytes, hipStream_t stream);
kvp_status kvp_launch_decode_step(const kvp_scorer* sc, const void* x_new, float* part,
                                  const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                                  const void* v_new, const float* s_in, int64_t ld_s, float* s_out,
                                  const float* tau, int* pos, const void* q, int B, int Hq,
                                  float sm_scale, float* out, void* ws, hipStream_t stream);
kvp_status kvp_launch_prefill_attn(const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                                   int T, int d, const uint32_t* keep_bits, const int* kept_idx,
                                   int window, float sm_scale, float* out, hipStream_t stream);
kvp_status kvp_launch_reset(const kvp_paged_kv* kv, const kvp_ring* ring, hipStream_t stream);
kvp_status kvp_launch_clear_error(const kvp_paged_kv* kv, hipStream_t stream);

namespace {

constexpr int64_t kMaxTokens = (int64_t)1 << 30;

bool is_kv_dtype(int32_t dt) { return dt == KVP_F32 || dt == KVP_BF16; }

kvp_status check_kv(const kvp_paged_kv* kv) {
  if (!kv) return KVP_E_ARG;
  if (!is_kv_dtype(kv->dtype)) return KVP_E_DTYPE;
  if (kv->num_pairs <= 0 || kv->num_pairs > 65535) return KVP_E_ARG;
  if (kv->head_dim != 64 && kv->head_dim != 128) return KVP_E_UNSUPPORTED;
  if (kv->num_pages < 0 || kv->max_pages_per_pair <= 0) return KVP_E_ARG;
  if (!kv->k_pages || !kv->v_pages || !kv->page_pos || !kv->block_table || !kv->length ||
      !kv->page_top || !kv->err)
    return KVP_E_ARG;
  if (kv->num_pages8 < 0) return KVP_E_ARG;
  if (kv->num_pages8 > 0) {
    if (kv->max_pages8_per_pair <= 0) return KVP_E_ARG;
    if (kv->lp_bits != 0 && kv->lp_bits != KVP_LP_INT8 && kv->lp_bits != KVP_LP_INT4 &&
        kv->lp_bits != KVP_LP_FP8_E4M3)
      return KVP_E_ARG;
    if (!kv->k8_pages || !kv->v8_pages || !kv->k8_scale || !kv->v8_scale || !kv->page8_pos ||
        !kv->block_table8 || !kv->length8 || !kv->page8_top)
      return KVP_E_ARG;
  }
  return KVP_OK;
}

kvp_status check_ring(const kvp_ring* r) {
  if (!r) return KVP_OK;
  if (r->window <= 0 || r->window % KVP_PAGE != 0) return KVP_E_ARG;
  if (r->window > 1024) return KVP_E_UNSUPPORTED;
  if (!r->k || !r->v || !r->score || !r->pos) return KVP_E_ARG;
  return KVP_OK;
}

}  // namespace

extern "C" const char* kvp_status_str(kvp_status s) {
  switch (s) {
    case KVP_OK: return "KVP_OK";
    case KVP_E_ARG: return "KVP_E_ARG: invalid argument";
    case KVP_E_DTYPE: return "KVP_E_DTYPE: unsupported dtype combination";
    case KVP_E_WORKSPACE: return "KVP_E_WORKSPACE: workspace missing or too small";
    case KVP_E_CAPACITY: return "KVP_E_CAPACITY: page pool or block table exhausted";
    case KVP_E_HIP: return "KVP_E_HIP: HIP runtime error";
    case KVP_E_UNSUPPORTED: return "KVP_E_UNSUPPORTED: not implemented for these sizes";
  }
  return "KVP_E_UNKNOWN";
}

extern "C" const char* kvp_version(void) { return "libkvp 0.1.0 gfx950"; }

extern "C" kvp_status kvp_score(const kvp_scorer* sc, const void* hidden, int32_t hdtype, int32_t B,
                                int32_t T, float* scores, int64_t ld_s, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (!sc || !hidden || !scores || !sc->w1) return KVP_E_ARG;
  if (B <= 0 || T <= 0 || ld_s < T || sc->hidden <= 0) return KVP_E_ARG;
  if ((int64_t)B * T > kMaxTokens) return KVP_E_ARG;
  if (sc->n_kv_heads <= 0 || sc->n_kv_heads > 16) return KVP_E_UNSUPPORTED;
  if (!is_kv_dtype(hdtype) || hdtype != sc->wdtype) return KVP_E_DTYPE;
  if (sc->kind == KVP_SCORER_LINEAR) {
    if (hdtype == KVP_BF16 && sc->hidden % 32 != 0) return KVP_E_UNSUPPORTED;
  } else if (sc->kind == KVP_SCORER_MLP) {
    if (hdtype != KVP_BF16) return KVP_E_DTYPE;
    if (!sc->w2) return KVP_E_ARG;
    if (sc->inner <= 0 || sc->inner % 256 != 0 || sc->hidden % 64 != 0) return KVP_E_UNSUPPORTED;
  } else {
    return KVP_E_ARG;
  }
  const size_t need = kvp_score_workspace_size(sc, B, T);
  if (need > 0 && (!ws || ws_bytes < need)) return KVP_E_WORKSPACE;
  return kvp_launch_score(sc, hidden, B, T, scores, ld_s, ws, stream);
}

static kvp_status select_common(const float* scores, int32_t B, int32_t Hkv, int32_t T, int64_t ld_s,
                                float tau, const float* tau_dev, int32_t recent, uint32_t* keep_bits,
                                int32_t* kept_idx, int32_t* kept_count, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (!scores || !keep_bits || !kept_idx || !kept_count) return KVP_E_ARG;
  if (B <= 0 || Hkv <= 0 || T <= 0 || ld_s < T || recent < 0) return KVP_E_ARG;
  if ((int64_t)B * Hkv > 65535 || T > kMaxTokens) return KVP_E_ARG;
  if (!ws || ws_bytes < kvp_select_workspace_size(B, Hkv, T)) return KVP_E_WORKSPACE;
  return kvp_launch_select(scores, B * Hkv, T, ld_s, tau, tau_dev, recent, keep_bits, kept_idx,
                           kept_count, ws, stream);
}

extern "C" kvp_status kvp_select(const float* scores, int32_t B, int32_t Hkv, int32_t T,
                                 int64_t ld_s, float tau, int32_t recent, uint32_t* keep_bits,
                                 int32_t* kept_idx, int32_t* kept_count, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  return select_common(scores, B, Hkv, T, ld_s, tau, nullptr, recent, keep_bits, kept_idx,
                       kept_count, ws, ws_bytes, stream);
}

extern "C" kvp_status kvp_select_dev_tau(const float* scores, int32_t B, int32_t Hkv, int32_t T,
                                         int64_t ld_s, const float* tau, int32_t recent,
                                         uint32_t* keep_bits, int32_t* kept_idx,
                                         int32_t* kept_count, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  if (!tau) return KVP_E_ARG;
  return select_common(scores, B, Hkv, T, ld_s, 0.0f, tau, recent, keep_bits, kept_idx, kept_count,
                       ws, ws_bytes, stream);
}

extern "C" kvp_status kvp_threshold(const float* scores, int32_t B, int32_t Hkv, int32_t T,
                                    int64_t ld_s, double q, float* tau_out, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  if (!scores || !tau_out) return KVP_E_ARG;
  if (B <= 0 || Hkv <= 0 || T <= 0 || ld_s < T) return KVP_E_ARG;
  if (!(q >= 0.0 && q <= 1.0)) return KVP_E_ARG;  // also rejects NaN
  if ((int64_t)B * Hkv > 65535 || (int64_t)B * Hkv * T > 0xffffffffLL) return KVP_E_UNSUPPORTED;
  if (!ws || ws_bytes < kvp_threshold_workspace_size()) return KVP_E_WORKSPACE;
  return kvp_launch_threshold(scores, B * Hkv, T, ld_s, q, tau_out, ws, stream);
}

extern "C" kvp_status kvp_compact(const void* k, const void* v, int32_t dtype, int32_t B,
                                  int32_t Hkv, int32_t T, int32_t d, const int32_t* kept_idx,
                                  const int32_t* kept_count, const float* scores, int64_t ld_s,
                                  int32_t mode, const kvp_paged_kv* kv, const kvp_ring* ring, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  kvp_status st = check_kv(kv);
  if (st != KVP_OK) return st;
  if ((st = check_ring(ring)) != KVP_OK) return st;
  if (!k || !v || !kept_idx || !kept_count) return KVP_E_ARG;
  if (B <= 0 || Hkv <= 0 || T <= 0 || T > kMaxTokens) return KVP_E_ARG;
  if ((int64_t)B * Hkv != kv->num_pairs) return KVP_E_ARG;
  if (d != kv->head_dim) return KVP_E_ARG;
  if (dtype != kv->dtype) return KVP_E_DTYPE;
  if (mode != KVP_COMPACT_EVICT && mode != KVP_COMPACT_DEMOTE_INT8) return KVP_E_ARG;
  if (mode == KVP_COMPACT_DEMOTE_INT8 && kv->num_pages8 <= 0) return KVP_E_ARG;
  if (ring && (!scores || ld_s < T)) return KVP_E_ARG;
  if (!ws || ws_bytes < kvp_compact_workspace_size(B, Hkv)) return KVP_E_WORKSPACE;
  return kvp_launch_compact(k, v, kv->num_pairs, T, d, kept_idx, kept_count, scores, ld_s,
                            mode == KVP_COMPACT_DEMOTE_INT8, kv, ring, ws, stream);
}

static kvp_status step_common(const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                              const void* v_new, int32_t dtype, const float* s_new, int64_t ld_s,
                              float tau, const float* tau_dev, int32_t p, int32_t* pos_dev,
                              hipStream_t stream) {
  kvp_status st = check_kv(kv);
  if (st != KVP_OK) return st;
  if (!ring) return KVP_E_ARG;
  if ((st = check_ring(ring)) != KVP_OK) return st;
  if (!k_new || !v_new || !s_new || ld_s < 1 || p < 0) return KVP_E_ARG;
  if (dtype != kv->dtype) return KVP_E_DTYPE;
  return kvp_launch_step_delayed(kv, ring, k_new, v_new, s_new, ld_s, tau, tau_dev, p, pos_dev,
                                 stream);
}

extern "C" kvp_status kvp_step_delayed(const kvp_paged_kv* kv, const kvp_ring* ring,
                                       const void* k_new, const void* v_new, int32_t dtype,
                                       const float* s_new, int64_t ld_s, float tau, int32_t p,
                                       hipStream_t stream) {
  return step_common(kv, ring, k_new, v_new, dtype, s_new, ld_s, tau, nullptr, p, nullptr, stream);
}

extern "C" kvp_status kvp_step_delayed_dev(const kvp_paged_kv* kv, const kvp_ring* ring,
                                           const void* k_new, const void* v_new, int32_t dtype,
                                           const float* s_new, int64_t ld_s, const float* tau,
                                           int32_t* pos, hipStream_t stream) {
  if (!tau || !pos) return KVP_E_ARG;
  return step_common(kv, ring, k_new, v_new, dtype, s_new, ld_s, 0.0f, tau, 0, pos, stream);
}

extern "C" kvp_status kvp_score_step_delayed(const kvp_scorer* sc, const void* hidden_new,
                                             int32_t hdtype, const kvp_paged_kv* kv,
                                             const kvp_ring* ring, const void* k_new,
                                             const void* v_new, int32_t dtype, float* s_new,
                                             const float* tau, int32_t* pos, void* ws,
                                             size_t ws_bytes, hipStream_t stream) {
  kvp_status st = check_kv(kv);
  if (st != KVP_OK) return st;
  if (!ring) return KVP_E_ARG;
  if ((st = check_ring(ring)) != KVP_OK) return st;
  if (!sc || !hidden_new || !sc->w1 || !k_new || !v_new || !tau || !pos) return KVP_E_ARG;
  if (sc->n_kv_heads <= 0 || sc->n_kv_heads > 16 || kv->num_pairs % sc->n_kv_heads != 0)
    return KVP_E_ARG;
  if (!is_kv_dtype(hdtype) || hdtype != sc->wdtype) return KVP_E_DTYPE;
  if (dtype != kv->dtype) return KVP_E_DTYPE;
  if (sc->kind == KVP_SCORER_LINEAR) {
    // rows are read in 16-byte pieces
    const int elt = hdtype == KVP_BF16 ? 2 : 4;
    if (sc->hidden <= 0 || sc->hidden % (16 / elt) != 0) return KVP_E_UNSUPPORTED;
    if (((uintptr_t)hidden_new | (uintptr_t)sc->w1) & 15) return KVP_E_ARG;
    return kvp_launch_step_delayed(kv, ring, k_new, v_new, nullptr, 1, 0.0f, tau, 0, pos, stream,
                                   sc, hidden_new, s_new);
  }
  if (sc->kind != KVP_SCORER_MLP) return KVP_E_ARG;
  const int B = kv->num_pairs / sc->n_kv_heads;
  if (!sc->w2) return KVP_E_ARG;
  if (sc->hidden <= 0 || sc->inner <= 0 || !kvp_score_small_mlp_ok(sc, B)) return KVP_E_UNSUPPORTED;
  // the finish reads b1, W2 rows and the partial sums in 16-byte pieces
  if (((uintptr_t)ws | (uintptr_t)sc->b1 | (uintptr_t)sc->w2) & 15) return KVP_E_ARG;
  if (!ws || ws_bytes < kvp_score_workspace_size(sc, B, 1)) return KVP_E_WORKSPACE;
  float* part = reinterpret_cast<float*>(ws);
  if ((st = kvp_launch_score_small_partials(sc, hidden_new, B, part, stream)) != KVP_OK) return st;
  return kvp_launch_step_delayed(kv, ring, k_new, v_new, nullptr, 1, 0.0f, tau, 0, pos, stream,
                                 sc, hidden_new, s_new, part);
}

namespace {

// Shape and dtype rules shared by both decode-attention entry points.
kvp_status check_decode_attn(const void* q, int32_t qdtype, int32_t B, int32_t Hq,
                             const kvp_paged_kv* kv, const kvp_ring* ring, const float* out) {
  kvp_status st = check_kv(kv);
  if (st != KVP_OK) return st;
  if ((st = check_ring(ring)) != KVP_OK) return st;
  if (!q || !out) return KVP_E_ARG;
  if (B <= 0 || Hq <= 0 || kv->num_pairs % B != 0) return KVP_E_ARG;
  const int Hkv = kv->num_pairs / B;
  if (Hq % Hkv != 0) return KVP_E_ARG;
  if (Hq / Hkv > 16) return KVP_E_UNSUPPORTED;
  if (qdtype != kv->dtype) return KVP_E_DTYPE;
  if (kv->num_pages8 > 0 && kv->dtype != KVP_BF16) return KVP_E_DTYPE;
  return KVP_OK;
}

}  // namespace

extern "C" kvp_status kvp_decode_attn(const void* q, int32_t qdtype, int32_t B, int32_t Hq,
                                      const kvp_paged_kv* kv, const kvp_ring* ring, float sm_scale,
                                      float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const kvp_status st = check_decode_attn(q, qdtype, B, Hq, kv, ring, out);
  if (st != KVP_OK) return st;
  if (!ws || ws_bytes < kvp_decode_attn_workspace_size(B, Hq, kv->num_pairs, kv->head_dim))
    return KVP_E_WORKSPACE;
  if (((uintptr_t)ws) & 255) return KVP_E_ARG;
  return kvp_launch_decode_attn(q, B, Hq, kv, ring, sm_scale, out, ws, ws_bytes, stream);
}

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

extern "C" size_t kvp_decode_step_workspace_size(const kvp_scorer* sc, int32_t B, int32_t Hq,
                                                 int32_t num_pairs, int32_t head_dim) {
  const size_t attn = kvp_decode_attn_workspace_size(B, Hq, num_pairs, head_dim);
  if (attn == 0) return 0;
  const bool mlp = sc && sc->kind == KVP_SCORER_MLP;
  return align256(attn) + (mlp ? kvp_score_workspace_size(sc, B, 1) : 0);
}

extern "C" kvp_status kvp_decode_step(const kvp_scorer* sc, const void* hidden_new, int32_t hdtype,
                                      const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                                      const void* v_new, const float* s_in, int64_t ld_s, float* s_out,
                                      const float* tau, int32_t* pos, const void* q, int32_t qdtype,
                                      int32_t B, int32_t Hq, float sm_scale, float* out, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  kvp_status st = check_decode_attn(q, qdtype, B, Hq, kv, ring, out);
  if (st != KVP_OK) return st;
  if (!ring) return KVP_E_ARG;
  if (kv->dtype != KVP_BF16 || kv->num_pages8 > 0) return KVP_E_UNSUPPORTED;
  if (!k_new || !v_new || !tau || !pos) return KVP_E_ARG;
  // the new token's K row and V values are read in 16-byte pieces
  if (((uintptr_t)k_new | (uintptr_t)v_new) & 15) return KVP_E_ARG;
  const int Hkv = kv->num_pairs / B;
  float* part = nullptr;
  if (!sc) {
    if (!s_in || ld_s < 1) return KVP_E_ARG;
  } else {
    if (!hidden_new || !sc->w1) return KVP_E_ARG;
    if (sc->n_kv_heads != Hkv) return KVP_E_ARG;
    if (!is_kv_dtype(hdtype) || hdtype != sc->wdtype) return KVP_E_DTYPE;
    if (sc->kind == KVP_SCORER_LINEAR) {
      const int elt = hdtype == KVP_BF16 ? 2 : 4;
      if (sc->hidden <= 0 || sc->hidden % (16 / elt) != 0) return KVP_E_UNSUPPORTED;
      if (((uintptr_t)hidden_new | (uintptr_t)sc->w1) & 15) return KVP_E_ARG;
    } else if (sc->kind == KVP_SCORER_MLP) {
      if (!sc->w2) return KVP_E_ARG;
      if (sc->hidden <= 0 || sc->inner <= 0 || !kvp_score_small_mlp_ok(sc, B)) return KVP_E_UNSUPPORTED;
      if (((uintptr_t)sc->b1 | (uintptr_t)sc->w2) & 15) return KVP_E_ARG;
    } else {
      return KVP_E_ARG;
    }
  }
  if (!ws || ws_bytes < kvp_decode_step_workspace_size(sc, B, Hq, kv->num_pairs, kv->head_dim))
    return KVP_E_WORKSPACE;
  if (((uintptr_t)ws) & 255) return KVP_E_ARG;
  if (sc && sc->kind == KVP_SCORER_MLP) {
    float* pws = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) +
                                          align256(kvp_decode_attn_workspace_size(B, Hq, kv->num_pairs,
                                                                                  kv->head_dim)));
    part = pws;  // written by the attention's stream kernel, summed by its merge kernel
  }
  return kvp_launch_decode_step(sc, sc ? hidden_new : nullptr, part, kv, ring, k_new, v_new,
                                sc ? nullptr : s_in, ld_s, s_out, tau, pos, q, B, Hq, sm_scale, out, ws,
                                stream);
}

// Decode-attention scratch for callers that cannot allocate: a fixed array in device
// memory, one copy per GPU the library runs on, held until the process ends.  Host
// code never passes `scratch` itself to a kernel (on the host it is only a stand-in
// for the symbol); it uses the device address looked up once per device below.
static __device__ __align__(256) unsigned char scratch[KVP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices];  // device address of `scratch`, per device id

// Device address of `scratch` on `dev`, which must be the current device.  The first
// call on a device looks it up; later calls return the cached address.
kvp_status scratch_address(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxScratchDevices) return KVP_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVP_E_HIP;
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return KVP_OK;
}

}  // namespace

extern "C" kvp_status kvp_decode_attn_noalloc(const void* q, int32_t qdtype, int32_t B, int32_t Hq,
                                              const kvp_paged_kv* kv, const kvp_ring* ring,
                                              float sm_scale, float* out, hipStream_t stream) {
  const kvp_status st = check_decode_attn(q, qdtype, B, Hq, kv, ring, out);
  if (st != KVP_OK) return st;
  const size_t need = kvp_decode_attn_workspace_size(B, Hq, kv->num_pairs, kv->head_dim);
  if (need == 0 || need > (size_t)KVP_NOALLOC_SCRATCH_BYTES) return KVP_E_WORKSPACE;
  int cur = -1, sdev = -1;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &sdev) != hipSuccess)
    return KVP_E_HIP;
  if (sdev != cur) return KVP_E_ARG;
  void* ws = nullptr;
  const kvp_status sa = scratch_address(cur, &ws);
  if (sa != KVP_OK) return sa;
  // Nothing in the scratch has to start at zero: the first kernel writes the page
  // prefix and every record before the merge kernel reads them.
  return kvp_launch_decode_attn(q, B, Hq, kv, ring, sm_scale, out, ws, need, stream);
}

extern "C" kvp_status kvp_prefill_attn(const void* q, const void* k, const void* v, int32_t dtype,
                                       int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t d,
                                       const uint32_t* keep_bits, const int32_t* kept_idx,
                                       int32_t window, float sm_scale, float* out, hipStream_t stream) {
  if (!q || !k || !v || !keep_bits || !kept_idx || !out) return KVP_E_ARG;
  if (dtype != KVP_BF16) return is_kv_dtype(dtype) ? KVP_E_UNSUPPORTED : KVP_E_DTYPE;
  if (B <= 0 || Hkv <= 0 || Hq <= 0 || T <= 0 || window < 0) return KVP_E_ARG;
  if (!(sm_scale > 0.0f) || sm_scale == __builtin_huge_valf()) return KVP_E_ARG;
  if (Hq % Hkv != 0) return KVP_E_ARG;
  const int g = Hq / Hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8 && g != 16) return KVP_E_UNSUPPORTED;
  if (d != 64 && d != 128) return KVP_E_UNSUPPORTED;
  if ((int64_t)B * Hkv > 65535 || T > kMaxTokens) return KVP_E_UNSUPPORTED;
  return kvp_launch_prefill_attn(q, k, v, B, Hq, Hkv, T, d, keep_bits, kept_idx, window, sm_scale, out,
                                 stream);
}

extern "C" kvp_status kvp_reset(const kvp_paged_kv* kv, const kvp_ring* ring, hipStream_t stream) {
  kvp_status st = check_kv(kv);
  if (st != KVP_OK) return st;
  if ((st = check_ring(ring)) != KVP_OK) return st;
  return kvp_launch_reset(kv, ring, stream);
}

extern "C" kvp_status kvp_clear_error(const kvp_paged_kv* kv, hipStream_t stream) {
  if (!kv || !kv->err) return KVP_E_ARG;
  return kvp_launch_clear_error(kv, stream);
}

extern "C" kvp_status kvp_check(const kvp_paged_kv* kv, hipStream_t stream) {
  if (!kv || !kv->err) return KVP_E_ARG;
  if (hipStreamSynchronize(stream) != hipSuccess) return KVP_E_HIP;
  int host_err = 0;
  if (hipMemcpy(&host_err, kv->err, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess)
    return KVP_E_HIP;
  return host_err ? KVP_E_CAPACITY : KVP_OK;
}
