// Internal helpers shared by the libkvp translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "kvp.h"

namespace kvp {

constexpr int PAGE = KVP_PAGE;
constexpr int WAVE = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even (NaN stays NaN):
// gfx950 converts in hardware (v_cvt_pk_bf16_f32), two values per instruction.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// a, b -> {bf16 hi parts (packed), bf16 parts of the remainders (packed)}: hi + lo
// keeps ~16 significant bits of each value for a bf16 MFMA operand.
__device__ __forceinline__ u32x2 split_bf16x2(float a, float b) {
  const uint32_t hi = pack_bf16x2(a, b);
  return u32x2{hi, pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u))};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16x16x32 bf16 MFMA, fp32 accumulate.  Operand A: lane l holds row (l % 16) and 8
// K-slots of group (l / 16); operand B: column (l % 16), same K-slot group; the result
// C[r][c] sits in lane c + 16 * (r / 4), element r % 4.  K-slot order within a group
// only has to agree between A and B, which every caller keeps.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Exact-form GELU, 0.5 a (1 + erf(a / sqrt 2)) (not the tanh approximation), with erf by
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erf(z) = 1 - P(t) exp(-z^2), P(t) = a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5,
// t = 1/(1 + p z), z >= 0, |error| <= 1.5e-7.  Since a erf(a / sqrt 2) = |a| erf(|a| / sqrt 2),
//   GELU(a) = max(a, 0) - 0.5 |a| P(t) exp(-a^2 / 2),   t = 1/(1 + (p / sqrt 2) |a|),
// with 1/sqrt 2, 0.5 and log2(e) folded into the constants; for a < 0 the small result
// comes out directly rather than as 1 + erf, a difference of two numbers near 1.
// Branch-free (it runs on every unit of every token: 11 VALU operations, one reciprocal,
// one exp2), and its error moves a score by ~1e-6 at most here.
__device__ __forceinline__ float gelu_erf(float a) {
  const float aa = fabsf(a);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, aa, 1.0f));
  float q = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
  q = fmaf(t, q, 0.5f * 1.421413741f);
  q = fmaf(t, q, 0.5f * -0.284496736f);
  q = fmaf(t, q, 0.5f * 0.254829592f);
  q *= t;  // 0.5 P(t)
  const float e = __builtin_amdgcn_exp2f(a * (a * (-0.5f * 1.4426950408889634f)));
  return fmaf(-aa * q, e, fmaxf(a, 0.0f));
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Inclusive scan of one int per lane across the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Number of set bits of a 64-bit wave mask below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// Exclusive scan over n ints held in LDS, by the whole block (blockDim.x threads,
// multiple of 64).  Returns the total.  `tmp` needs one int per wave.
__device__ inline int block_excl_scan_lds(int* data, int n, int* tmp) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wid = tid >> 6;
  const int nw = nt >> 6;
  int carry = 0;
  for (int base = 0; base < n; base += nt) {
    int i = base + tid;
    int v = (i < n) ? data[i] : 0;
    int inc = wave_incl_scan(v);
    if (lane == 63) tmp[wid] = inc;
    __syncthreads();
    int woff = 0;
    for (int w = 0; w < wid; ++w) woff += tmp[w];
    int tot = 0;
    for (int w = 0; w < nw; ++w) tot += tmp[w];
    __syncthreads();
    if (i < n) data[i] = carry + woff + inc - v;
    carry += tot;
  }
  __syncthreads();
  return carry;
}

// Exclusive scan over n ints held in LDS by the whole block: each thread scans a
// contiguous chunk serially, the chunk totals are scanned across the wave with
// shuffles and across waves through `wtot` (one int per wave).  Returns the total.
__device__ inline int block_scan_excl(int* data, int n, int* wtot) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wid = tid >> 6;
  const int nw = nt >> 6;
  const int per = (n + nt - 1) / nt;
  const int b0 = min(n, tid * per), b1 = min(n, b0 + per);
  int sum = 0;
  for (int i = b0; i < b1; ++i) sum += data[i];
  const int inc = wave_incl_scan(sum);
  if (lane == 63) wtot[wid] = inc;
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int t = wtot[w];
    off += (w < wid) ? t : 0;
    tot += t;
  }
  int run = off + inc - sum;
  for (int i = b0; i < b1; ++i) {
    const int v = data[i];
    data[i] = run;
    run += v;
  }
  __syncthreads();
  return tot;
}

// Binary search in an ascending array a[0..n]: largest s in [0, n) with a[s] <= x.
__device__ __forceinline__ int upper_segment(const int* a, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Symmetric code of x with the given fp32 scale: round half to even, clamp to
// +-qmax (127 for int8 codes, 7 for int4); a zero scale gives code 0.
__device__ __forceinline__ int quant_code(float x, float scale, float qmax = 127.0f) {
  if (scale == 0.0f) return 0;
  float y = rintf(x / scale);
  y = fminf(fmaxf(y, -qmax), qmax);
  return static_cast<int>(y);
}

// Low-precision pool code width (kvp_paged_kv::lp_bits; 0 means 8; the fp8 format has
// 8-bit codes, so it shares the int8 pool's layout).
__host__ __device__ inline int lp_bits_of(const kvp_paged_kv& kv) { return kv.lp_bits == 4 ? 4 : 8; }
__host__ __device__ inline bool lp_is_fp8(const kvp_paged_kv& kv) { return kv.lp_bits == KVP_LP_FP8_E4M3; }

// OCP FP8 E4M3 code of an fp32 value (1 sign, 4 exponent bits with bias 7, 3 mantissa
// bits; largest finite magnitude 448; exponent field 0 holds the subnormals m 2^-9):
// round to nearest, ties to even; magnitudes at or above 448 saturate to 448.
__device__ __forceinline__ uint32_t fp8_e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t c;
  if (!(a < 448.0f)) {
    c = 0x7Eu;
  } else if (a < 0x1p-6f) {
    c = static_cast<uint32_t>(rintf(a * 512.0f));  // 0..8 (8: the smallest normal)
  } else {
    const uint32_t ua = __float_as_uint(a);
    const uint32_t m = ua & 0x7fffffu, rem = m & 0xfffffu;
    uint32_t k = (((ua >> 23) - 120u) << 3) | (m >> 20);  // biased exponent 127 -> 7
    k += (rem > 0x80000u || (rem == 0x80000u && (k & 1u))) ? 1u : 0u;
    c = k < 0x7Eu ? k : 0x7Eu;
  }
  return sign | c;
}

// fp8 code of x for a row scale s = fp32(max |x| / 448): the code of the correctly
// rounded fp32 quotient; a zero scale (an all-zero row) gives code 0.
__device__ __forceinline__ uint32_t fp8_quant_code(float x, float scale) {
  return scale == 0.0f ? 0u : fp8_e4m3_code(x / scale);
}

}  // namespace kvp

#define KVP_LAUNCH_CHECK()                                   \
  do {                                                       \
    hipError_t e_ = hipGetLastError();                       \
    if (e_ != hipSuccess) return KVP_E_HIP;                  \
  } while (0)
