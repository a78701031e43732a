// One decode step of the recent-window ring with delayed eviction (gfx950).
//
// Method: DMS article (euno.news), "Delayed Eviction" -- a token flagged for eviction
// is not removed at once but kept in a short buffer for a fixed number of steps and
// deleted when that window expires.  KVzap digest (max5.ai), practical application --
// the most recent tokens are always kept and low-scoring ones are removed.
//
// The ring holds the last `window` positions of every pair (position t in slot
// t mod window).  Appending position p evicts position p - window from its slot (the
// per-pair work is step_pair in step_core.h).  One wave per pair; O(1) work.
#include "step_core.h"

namespace kvp {

template <typename E, int D>
__global__ __launch_bounds__(256) void step_delayed_kernel(StepArgs a) {
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int p = a.pos_dev ? a.pos_dev[0] : a.p;
  if (pair < a.kv.num_pairs) step_pair<E, D>(a, pair, p);
  // Device-resident position: every wave of the work-group has read it (above) before
  // the work-group counts itself here; the last of the work-groups to arrive advances
  // it and clears the count, so the next call (or graph replay) appends the next
  // position.  One count per work-group keeps the same-address atomics few.
  if (a.pos_dev) {
    __syncthreads();
    if (threadIdx.x == 0 && atomicAdd(&a.pos_dev[1], 1) == (int)gridDim.x - 1) {
      a.pos_dev[0] = p + 1;
      a.pos_dev[1] = 0;
    }
  }
}

}  // namespace kvp


using namespace kvp;

StepArgs kvp::make_step_args(const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                             const void* v_new, const float* s_new, int64_t ld_s, float tau,
                             const float* tau_dev, int p, int* pos_dev, const kvp_scorer* sc,
                             const void* x_new, float* s_out, const float* part) {
  StepArgs a;
  const bool mlp = sc && sc->kind == KVP_SCORER_MLP;
  a.x_new = mlp ? nullptr : x_new;
  a.w = sc ? sc->w1 : nullptr;
  a.bias = sc ? sc->b1 : nullptr;
  a.s_out = s_out;
  a.H = sc ? sc->hidden : 0;
  a.Hkv = sc ? sc->n_kv_heads : 1;
  a.x_bf16 = sc ? sc->wdtype == KVP_BF16 : 0;
  a.part = mlp ? part : nullptr;
  a.ksplit = mlp ? sc->hidden / 256 : 0;
  a.ntok = mlp ? kv->num_pairs / sc->n_kv_heads : 0;
  a.inner = mlp ? sc->inner : 0;
  a.b1 = mlp ? sc->b1 : nullptr;
  a.w2 = mlp ? sc->w2 : nullptr;
  a.b2 = mlp ? sc->b2 : nullptr;
  a.kv = *kv;
  a.ring = *ring;
  a.k_new = k_new;
  a.v_new = v_new;
  a.s_new = s_new;
  a.ld_s = ld_s;
  a.tau = tau;
  a.tau_dev = tau_dev;
  a.p = p;
  a.pos_dev = pos_dev;
  return a;
}

kvp_status kvp_launch_step_delayed(const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                                   const void* v_new, const float* s_new, int64_t ld_s, float tau,
                                   const float* tau_dev, int p, int* pos_dev, hipStream_t stream,
                                   const kvp_scorer* sc, const void* x_new, float* s_out,
                                   const float* part) {
  const StepArgs a = make_step_args(kv, ring, k_new, v_new, s_new, ld_s, tau, tau_dev, p, pos_dev, sc,
                                    x_new, s_out, part);
  const dim3 grid(cdiv(kv->num_pairs, 4));
  if (kv->dtype == KVP_BF16) {
    if (kv->head_dim == 64) hipLaunchKernelGGL((step_delayed_kernel<uint16_t, 64>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((step_delayed_kernel<uint16_t, 128>), grid, dim3(256), 0, stream, a);
  } else {
    if (kv->head_dim == 64) hipLaunchKernelGGL((step_delayed_kernel<float, 64>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((step_delayed_kernel<float, 128>), grid, dim3(256), 0, stream, a);
  }
  KVP_LAUNCH_CHECK();
  return KVP_OK;
}
