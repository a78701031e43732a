// Keep mask and ordered index lists (gfx950).
//
// Method: KVzap digest (max5.ai), key points, practical application -- entries whose
// score is low are removed and the most recent 128 tokens are always kept:
//   keep[p][t] = (s[p][t] >= tau) || (t >= T - recent).
//
// Two passes over tiles of 2048 tokens per pair:
//   1. each wave evaluates 64 tokens at a time, __ballot gives the 64-bit mask word
//      pair (stored as two u32 of keep_bits) and __popcll the tile's kept count;
//   2. each tile reads the counts of the tiles before it (exclusive prefix) and the
//      pair total, rebuilds the masks from keep_bits, and ranks every token with
//      mbcnt (kept rank) inside the wave and an LDS prefix across waves.  A kept
//      token t goes to kept_idx[rank]; an evicted one to kept_idx[count + t - rank].
#include "kvp_internal.h"

namespace kvp {

constexpr int SEL_TILE = 2048;
constexpr int SEL_THREADS = 256;
constexpr int SEL_GROUPS = SEL_TILE / SEL_THREADS;  // 64-token groups per wave

__global__ __launch_bounds__(SEL_THREADS) void select_bits_kernel(
    const float* __restrict__ scores, int T, int64_t ld_s, float tau_val, const float* tau_dev,
    int recent, uint32_t* __restrict__ bits, int nwords, int* __restrict__ tile_count, int ntiles) {
  const int pair = blockIdx.y, tile = blockIdx.x;
  const float tau = tau_dev ? tau_dev[0] : tau_val;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const float* s = scores + (int64_t)pair * ld_s;
  uint32_t* bw = bits + (int64_t)pair * nwords;
  const int first_recent = T - recent;  // recent >= 0, may be <= 0 (all recent)
  int cnt = 0;
  const int t_begin = tile * SEL_TILE + wid * (SEL_GROUPS * 64);
#pragma unroll
  for (int gi = 0; gi < SEL_GROUPS; ++gi) {
    const int t0 = t_begin + gi * 64;
    if (t0 >= T) break;
    const int t = t0 + lane;
    bool keep = false;
    if (t < T) keep = (s[t] >= tau) || (t >= first_recent);
    const uint64_t m = __ballot(keep);
    if (lane == 0) {
      bw[t0 >> 5] = static_cast<uint32_t>(m);
      if ((t0 >> 5) + 1 < nwords) bw[(t0 >> 5) + 1] = static_cast<uint32_t>(m >> 32);
    }
    cnt += __popcll(m);
  }
  __shared__ int red[SEL_THREADS / 64];
  if (lane == 0) red[wid] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0;
    for (int w = 0; w < SEL_THREADS / 64; ++w) c += red[w];
    tile_count[(int64_t)pair * ntiles + tile] = c;
  }
}

__global__ __launch_bounds__(SEL_THREADS) void select_scatter_kernel(
    const uint32_t* __restrict__ bits, int T, int nwords, const int* __restrict__ tile_count,
    int ntiles, int* __restrict__ kept_idx, int* __restrict__ kept_count) {
  const int pair = blockIdx.y, tile = blockIdx.x;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __shared__ int sh_before[SEL_THREADS / 64], sh_total[SEL_THREADS / 64], sh_w[SEL_THREADS / 64];

  int before = 0, total = 0;
  for (int i = threadIdx.x; i < ntiles; i += SEL_THREADS) {
    const int c = tile_count[(int64_t)pair * ntiles + i];
    total += c;
    if (i < tile) before += c;
  }
  before = wave_sum_i(before);
  total = wave_sum_i(total);

  const uint32_t* bw = bits + (int64_t)pair * nwords;
  uint64_t masks[SEL_GROUPS];
  int wcnt = 0;
  const int t_begin = tile * SEL_TILE + wid * (SEL_GROUPS * 64);
#pragma unroll
  for (int gi = 0; gi < SEL_GROUPS; ++gi) {
    const int t0 = t_begin + gi * 64;
    uint64_t m = 0;
    if (t0 < T) {
      const int w0 = t0 >> 5;
      m = bw[w0];
      if (w0 + 1 < nwords) m |= static_cast<uint64_t>(bw[w0 + 1]) << 32;
    }
    masks[gi] = m;
    wcnt += __popcll(m);
  }
  if (lane == 0) {
    sh_before[wid] = before;
    sh_total[wid] = total;
    sh_w[wid] = wcnt;
  }
  __syncthreads();
  int tb = 0, tt = 0, woff = 0;
  for (int w = 0; w < SEL_THREADS / 64; ++w) {
    tb += sh_before[w];
    tt += sh_total[w];
    if (w < wid) woff += sh_w[w];
  }
  int run = tb + woff;  // kept positions before this wave's first token
  int* out = kept_idx + (int64_t)pair * T;
#pragma unroll
  for (int gi = 0; gi < SEL_GROUPS; ++gi) {
    const int t0 = t_begin + gi * 64;
    if (t0 >= T) break;
    const int t = t0 + lane;
    const uint64_t m = masks[gi];
    const int r = run + lanes_below(m);
    if (t < T) {
      if ((m >> lane) & 1ull) out[r] = t;
      else out[tt + (t - r)] = t;
    }
    run += __popcll(m);
  }
  if (tile == 0 && threadIdx.x == 0) kept_count[pair] = tt;
}

// ---------------------------------------------------------------- helpers
__global__ void reset_kernel(kvp_paged_kv kv, kvp_ring ring, int has_ring) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = tid; i < kv.num_pairs; i += stride) {
    kv.length[i] = 0;
    if (kv.num_pages8 > 0) kv.length8[i] = 0;
  }
  if (tid == 0) {
    kv.page_top[0] = 0;
    if (kv.num_pages8 > 0) kv.page8_top[0] = 0;
  }
  if (has_ring) {
    const int64_t n = (int64_t)kv.num_pairs * ring.window;
    for (int64_t i = tid; i < n; i += stride) {
      ring.pos[i] = -1;
      ring.score[i] = 0.f;
    }
  }
}

__global__ void clear_error_kernel(int* err) { err[0] = 0; }

}  // namespace kvp

using namespace kvp;

extern "C" size_t kvp_select_workspace_size(int32_t B, int32_t Hkv, int32_t T) {
  if (B <= 0 || Hkv <= 0 || T <= 0) return 0;
  return (size_t)B * Hkv * cdiv(T, SEL_TILE) * sizeof(int);
}

kvp_status kvp_launch_select(const float* scores, int num_pairs, int T, int64_t ld_s, float tau,
                             const float* tau_dev, int recent, uint32_t* bits, int* kept_idx,
                             int* kept_count, void* ws, hipStream_t stream) {
  const int ntiles = cdiv(T, SEL_TILE);
  const int nwords = cdiv(T, 32);
  int* tile_count = reinterpret_cast<int*>(ws);
  dim3 grid(ntiles, num_pairs);
  hipLaunchKernelGGL(select_bits_kernel, grid, dim3(SEL_THREADS), 0, stream, scores, T, ld_s, tau,
                     tau_dev, recent, bits, nwords, tile_count, ntiles);
  KVP_LAUNCH_CHECK();
  hipLaunchKernelGGL(select_scatter_kernel, grid, dim3(SEL_THREADS), 0, stream, bits, T, nwords,
                     tile_count, ntiles, kept_idx, kept_count);
  KVP_LAUNCH_CHECK();
  return KVP_OK;
}

kvp_status kvp_launch_reset(const kvp_paged_kv* kv, const kvp_ring* ring, hipStream_t stream) {
  kvp_ring r;
  if (ring) r = *ring;
  else r = kvp_ring{};
  hipLaunchKernelGGL(reset_kernel, dim3(256), dim3(256), 0, stream, *kv, r, ring ? 1 : 0);
  KVP_LAUNCH_CHECK();
  return KVP_OK;
}

kvp_status kvp_launch_clear_error(const kvp_paged_kv* kv, hipStream_t stream) {
  hipLaunchKernelGGL(clear_error_kernel, dim3(1), dim3(1), 0, stream, kv->err);
  KVP_LAUNCH_CHECK();
  return KVP_OK;
}
