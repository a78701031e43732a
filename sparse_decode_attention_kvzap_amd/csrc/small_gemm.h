// Split-K first layer of the scorer for a handful of tokens (gfx950).
//
// Method: KVzap digest (max5.ai), key points -- the MLP surrogate scorer's first layer,
// x W1^T, for the new tokens of a decode step (one per sequence).  A GEMM tile per
// work-group would leave all but a few CUs idle and walk the whole K loop serially, so
// the contraction is split: slice (r, ks) contracts rows [16r, 16r+16) of W (zero past
// `rows`) with every token over K slice ks (SMALL_KSLICE wide) on MFMA, straight from
// global memory, into part[ks][token][row]; the consumer adds the slices in a fixed order
// and finishes the scorer.  Used by the scorer's own small-batch kernel and by the fused
// decode step, whose attention waves take the slices at kernel start.
#pragma once
#include "kvp_internal.h"

namespace kvp {

constexpr int SMALL_MAX_TOK = 64;
constexpr int SMALL_KSLICE = 256;

struct SmallGemm {
  const uint16_t* x;  // [ntok][H] bf16
  const uint16_t* w;  // [rows][H] bf16
  float* part;        // [H / SMALL_KSLICE][ntok][16 * rtiles]
  int rows, ntok, H, rtiles, ksplit;
};

// Slice t = (rt, ks), rt = t % rtiles, for NTT = ceil(ntok / 16) 16-token tiles.  Loads
// are unconditional (token rows clamped, rows of W past `rows` read row 0 and are
// zeroed) so a wave issues all of its loads before its MFMAs instead of waiting on each
// behind a branch.
template <int NTT>
__device__ __forceinline__ void small_gemm_slice(const SmallGemm& g, int t) {
  const int lane = threadIdx.x & 63, n = lane & 15, j = lane >> 4;
  const int rt = t % g.rtiles, ks = t / g.rtiles;
  const int row = rt * 16 + n;
  const bool rv = row < g.rows;
  const uint16_t* wr = g.w + (int64_t)(rv ? row : 0) * g.H + ks * SMALL_KSLICE + 8 * j;
  const uint16_t* xr[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int tok = min(tt * 16 + n, g.ntok - 1);
    xr[tt] = g.x + (int64_t)tok * g.H + ks * SMALL_KSLICE + 8 * j;
  }
  constexpr int NK = SMALL_KSLICE / 32;
  u32x4 wv[NK], xv[NK][NTT];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    wv[kk] = *reinterpret_cast<const u32x4*>(wr + 32 * kk);
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) xv[kk][tt] = *reinterpret_cast<const u32x4*>(xr[tt] + 32 * kk);
  }
  f32x4 acc[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const u32x4 wk = rv ? wv[kk] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[tt] = mfma16x16x32(as_bf16x8(wk), as_bf16x8(xv[kk][tt]), acc[tt]);
  }
  // acc[tt][i] = C[row 16rt + 4j + i][token 16tt + n]
  const int rpad = g.rtiles * 16;
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int tok = tt * 16 + n;
    if (tok < g.ntok) {
      float* dst = g.part + ((int64_t)ks * g.ntok + tok) * rpad + rt * 16 + 4 * j;
      *reinterpret_cast<f32x4*>(dst) = acc[tt];
    }
  }
}

// Host: the contraction of `rows` rows of the scorer's W1 with ntok hidden rows.
SmallGemm small_gemm_of(const kvp_scorer* sc, const void* hidden, int ntok, int rows, float* part);

// Slices first, first + stride, ... of the whole contraction, by one wave.
__device__ __forceinline__ void small_gemm_slices(const SmallGemm& g, int first, int stride) {
  const int ns = g.rtiles * g.ksplit;
  const int ntt = (g.ntok + 15) / 16;
  for (int t = first; t < ns; t += stride) {
    if (ntt == 1) small_gemm_slice<1>(g, t);
    else if (ntt == 2) small_gemm_slice<2>(g, t);
    else if (ntt == 3) small_gemm_slice<3>(g, t);
    else small_gemm_slice<4>(g, t);
  }
}

}  // namespace kvp
