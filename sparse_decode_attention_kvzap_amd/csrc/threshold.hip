// On-device threshold calibration: tau = a quantile of all scores (gfx950).
//
// Method: KVzap digest (max5.ai), key points -- entries whose score falls below a
// threshold are removed, so keeping a fraction k of the entries means thresholding at
// the (1 - k) quantile of the scores.  The quantile follows numpy's default "linear"
// rule: with N scores sorted ascending as a[0..N-1] and v = (N - 1) q, the result is
// a[floor v] interpolated towards a[floor v + 1] by the fractional part (the last
// element when v >= N - 1), the interpolation done in fp64 exactly as numpy writes it,
// and the result rounded to fp32.  Any NaN score makes the result NaN.
//
// The two order statistics are found exactly by a three-pass radix select over the
// scores' order-preserving 32-bit keys (11, 11 and 10 bits, most significant first).
// Pass p histograms the keys that match the digits chosen so far (one LDS histogram
// per work-group, merged with device-scope atomics into one of 8 global copies, which
// keeps the hottest bins of a peaked score distribution from serialising every
// work-group on one address); a one-work-group pick kernel then sums the copies, finds
// the bin holding each target rank and appends it to the prefix.  Each pass has its own
// histograms, all cleared by one kernel up front.  The two ranks share a histogram
// while their prefixes agree.
#include "kvp_internal.h"

namespace kvp {

constexpr int THR_BINS = 2048;
constexpr int THR_THREADS = 256;
constexpr int THR_CHUNK = 4096;  // scores per work-group and row (16 per thread)
constexpr int THR_COPIES = 8;    // global histogram copies
constexpr int THR_HIST = 3 * THR_COPIES * 2 * THR_BINS;  // [pass][copy][target][bin]

struct ThrState {
  uint32_t prefix[2];  // key digits chosen so far for ranks r1, r2
  uint32_t rank[2];    // remaining rank inside the chosen prefix
  uint32_t nan_count;
  uint32_t pad[11];
};

// Workspace: ThrState (64 bytes), then hist[3][THR_COPIES][2][THR_BINS] u32.
__device__ __forceinline__ ThrState* thr_state(void* ws) { return reinterpret_cast<ThrState*>(ws); }
__device__ __forceinline__ uint32_t* thr_hist(void* ws, int pass) {
  return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) + sizeof(ThrState)) +
         pass * THR_COPIES * 2 * THR_BINS;
}


// Order-preserving key: negative floats have all bits flipped, non-negative ones only
// the sign bit, so unsigned key order is float order (-0 just below +0).
__device__ __forceinline__ uint32_t float_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// pass p: digit width and position
__device__ __forceinline__ int thr_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ int thr_width(int pass) { return pass == 2 ? 10 : 11; }

__global__ __launch_bounds__(THR_THREADS) void thr_init_kernel(void* ws, uint32_t r1, uint32_t r2) {
  uint32_t* h = thr_hist(ws, 0);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < THR_HIST; i += gridDim.x * blockDim.x) h[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ThrState* s = thr_state(ws);
    s->prefix[0] = s->prefix[1] = 0u;
    s->rank[0] = r1;
    s->rank[1] = r2;
    s->nan_count = 0u;
  }
}

// One work-group after pass p: for each target, sum the copies, find the bin whose
// cumulative count range holds the remaining rank (target 1 reads target 0's
// histogram while the prefixes agree) and append it to the prefix; after the last
// pass, numpy's lerp in fp64.
__global__ __launch_bounds__(THR_THREADS) void thr_pick_kernel(int pass, void* ws, double gamma,
                                                               float* tau_out) {
  __shared__ uint32_t wsum[THR_THREADS / 64];
  __shared__ uint32_t found[2], rem[2];
  constexpr int PER = THR_BINS / THR_THREADS;  // 8 bins per thread
  ThrState* st = thr_state(ws);
  const uint32_t* gh = thr_hist(ws, pass);
  const uint32_t P0 = st->prefix[0], P1 = st->prefix[1];
  const bool two = P1 != P0;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t cc[2][PER];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < PER; ++i) cc[t][i] = 0u;
#pragma unroll
  for (int cp = 0; cp < THR_COPIES; ++cp)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < PER; ++i) cc[t][i] += gh[(cp * 2 + t) * THR_BINS + tid * PER + i];
  for (int t = 0; t < 2; ++t) {
    const uint32_t rank = st->rank[t];
    const int ht = (t == 1 && two) ? 1 : 0;
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) sum += cc[ht][i];
    // exclusive scan of the per-thread sums (bins are in thread order)
    uint32_t incl = sum;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    uint32_t cum = incl - sum;
    for (int w = 0; w < wid; ++w) cum += wsum[w];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t c = cc[ht][i];
      if (c && cum <= rank && rank < cum + c) {
        found[t] = static_cast<uint32_t>(tid * PER + i);
        rem[t] = rank - cum;
      }
      cum += c;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int width = thr_width(pass);
    uint32_t pf[2];
    for (int t = 0; t < 2; ++t) {
      pf[t] = (st->prefix[t] << width) | found[t];
      st->prefix[t] = pf[t];
      st->rank[t] = rem[t];
    }
    if (pass == 2) {
      // a + (b - a) t, or b - (b - a)(1 - t) when t >= 0.5
      const double a = static_cast<double>(key_float(pf[0]));
      const double b = static_cast<double>(key_float(pf[1]));
      const double diff = b - a;
      double r = a + diff * gamma;
      if (gamma >= 0.5) r = b - diff * (1.0 - gamma);
      if (st->nan_count) r = __builtin_nan("");
      tau_out[0] = static_cast<float>(r);
    }
  }
}

// grid (ceil(T / THR_CHUNK), rows)
__global__ __launch_bounds__(THR_THREADS) void thr_hist_kernel(const float* __restrict__ scores, int T,
                                                               int64_t ld_s, int pass, void* ws) {
  __shared__ uint32_t lh[2][THR_BINS];
  const ThrState* st = thr_state(ws);
  const uint32_t P0 = st->prefix[0], P1 = st->prefix[1];
  const bool two = P1 != P0;
  const int shift = thr_shift(pass), width = thr_width(pass);
  const int hi = shift + width;  // bits above the digit form the prefix
  const uint32_t mask = (1u << width) - 1u;
  for (int i = threadIdx.x; i < 2 * THR_BINS; i += blockDim.x) (&lh[0][0])[i] = 0u;
  const float* row = scores + (int64_t)blockIdx.y * ld_s;
  const int t0 = blockIdx.x * THR_CHUNK;
  const int t1 = min(T, t0 + THR_CHUNK);
  // all 16 loads of a thread in flight (clamped, so none sits behind a branch)
  constexpr int EPT = THR_CHUNK / THR_THREADS;
  float f[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) f[i] = row[min(t0 + (int)threadIdx.x + i * THR_THREADS, t1 - 1)];
  __syncthreads();  // LDS histogram cleared
  uint32_t nans = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    if (t0 + (int)threadIdx.x + i * THR_THREADS >= t1) continue;
    if (f[i] != f[i]) {
      ++nans;
      continue;
    }
    const uint32_t k = float_key(f[i]);
    const uint32_t d = (k >> shift) & mask;
    const uint32_t pre = (hi >= 32) ? 0u : (k >> hi);
    if (pre == P0) atomicAdd(&lh[0][d], 1u);
    else if (two && pre == P1) atomicAdd(&lh[1][d], 1u);
  }
  __syncthreads();
  uint32_t* gh = thr_hist(ws, pass) + ((blockIdx.y * gridDim.x + blockIdx.x) % THR_COPIES) * 2 * THR_BINS;
  for (int i = threadIdx.x; i < 2 * THR_BINS; i += blockDim.x) {
    const uint32_t c = (&lh[0][0])[i];
    if (c) atomicAdd(gh + i, c);
  }
  if (pass == 0) {
    const int n = wave_sum_i(static_cast<int>(nans));
    if ((threadIdx.x & 63) == 0 && n) atomicAdd(&thr_state(ws)->nan_count, static_cast<uint32_t>(n));
  }
}

}  // namespace kvp

using namespace kvp;

extern "C" size_t kvp_threshold_workspace_size(void) {
  return sizeof(ThrState) + THR_HIST * sizeof(uint32_t);
}

kvp_status kvp_launch_threshold(const float* scores, int rows, int T, int64_t ld_s, double q,
                                float* tau_out, void* ws, hipStream_t stream) {
  // numpy "linear": virtual index v = (N - 1) q; the neighbours floor(v), floor(v) + 1,
  // or the last element (twice) when v >= N - 1; weight v - floor(v) (v + 1 in the
  // last case, which numpy's lerp turns into the last element itself).
  const double n = static_cast<double>(rows) * static_cast<double>(T);
  const double v = (n - 1.0) * q;
  uint32_t r1, r2;
  double gamma;
  if (v >= n - 1.0) {
    r1 = r2 = static_cast<uint32_t>(n - 1.0);
    gamma = v - (-1.0);
  } else {
    const double fl = floor(v);
    r1 = static_cast<uint32_t>(fl);
    r2 = r1 + 1u;
    gamma = v - fl;
  }
  hipLaunchKernelGGL(thr_init_kernel, dim3(cdiv(THR_HIST, 4 * THR_THREADS)), dim3(THR_THREADS), 0, stream,
                     ws, r1, r2);
  KVP_LAUNCH_CHECK();
  const dim3 grid(cdiv(T, THR_CHUNK), rows);
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(thr_hist_kernel, grid, dim3(THR_THREADS), 0, stream, scores, T, ld_s, pass, ws);
    KVP_LAUNCH_CHECK();
    hipLaunchKernelGGL(thr_pick_kernel, dim3(1), dim3(THR_THREADS), 0, stream, pass, ws, gamma, tau_out);
    KVP_LAUNCH_CHECK();
  }
  return KVP_OK;
}
