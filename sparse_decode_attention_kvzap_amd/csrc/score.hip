// Surrogate importance scorers (gfx950).
//
// Method: KVzap digest (max5.ai), key points -- a small surrogate model predicts each
// cache entry's importance directly from the hidden states, as a single linear layer
// (KVzap-Linear) or a two-layer MLP (KVzap-MLP); the memory/compute bullet puts their
// cost at ~0.02% and ~1.1% of the model's linear-projection FLOPs.
//
// Kernels:
//   score_linear_f32   VALU, one thread per (token, head); small fp32 workloads.
//   score_linear_bf16  16x16x32 bf16 MFMA: S[16 tok x 16 heads] per tile, HBM-bound
//                      streaming of the hidden rows (W stays in L2).
//   score_mlp_bf16     LDS-tiled bf16 MFMA GEMM computing A^T = W1 . X^T for a tile of
//                      256 inner units x 256 tokens; the epilogue adds b1, applies the
//                      exact erf GELU in fp32 and contracts with W2 on MFMA.  The GELU
//                      output u is fed to that second MFMA straight from the
//                      accumulator registers (the 16x16 result layout of two stacked
//                      tiles is a valid B-operand layout under a K-slot permutation,
//                      which W2's A operand follows), split into bf16 hi+lo parts, and
//                      W2 likewise, so the 512-term sum keeps ~16 significant bits per
//                      term.  Each 256-unit slice writes a partial score; a small finish
//                      kernel adds the slices in a fixed order plus b2.
#include "kvp_internal.h"
#include "small_gemm.h"

namespace kvp {

// ------------------------------------------------------------------ linear fp32
__global__ __launch_bounds__(256) void score_linear_f32_kernel(const float* __restrict__ X,
                                                               const float* __restrict__ W,
                                                               const float* __restrict__ bias,
                                                               int ntok, int H, int Hkv, int T,
                                                               float* __restrict__ scores,
                                                               int64_t ld_s) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)ntok * Hkv) return;
  const int tok = static_cast<int>(idx / Hkv), h = static_cast<int>(idx % Hkv);
  const float* x = X + (int64_t)tok * H;
  const float* w = W + (int64_t)h * H;
  float acc = 0.f;
  for (int i = 0; i < H; ++i) acc = fmaf(x[i], w[i], acc);
  if (bias) acc += bias[h];
  const int b = tok / T, t = tok % T;
  scores[((int64_t)b * Hkv + h) * ld_s + t] = acc;
}

// ------------------------------------------------------------------ linear bf16
constexpr int LIN_TILES = 4;  // 16-token tiles per wave
constexpr int LIN_U = 4;      // K-steps per load batch

__global__ __launch_bounds__(256) void score_linear_bf16_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, const float* __restrict__ bias,
    int ntok, int H, int Hkv, int T, float* __restrict__ scores, int64_t ld_s) {
  const int lane = threadIdx.x & 63, n = lane & 15, j = lane >> 4;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t tok0 = gw * (16 * LIN_TILES);
  if (tok0 >= ntok) return;
  const uint16_t* xr[LIN_TILES];
#pragma unroll
  for (int tt = 0; tt < LIN_TILES; ++tt) {
    int64_t tok = tok0 + 16 * tt + n;
    if (tok >= ntok) tok = ntok - 1;
    xr[tt] = X + tok * H + 8 * j;
  }
  const bool hv = n < Hkv;
  const uint16_t* wr = W + (int64_t)(hv ? n : 0) * H + 8 * j;
  f32x4 acc[LIN_TILES];
#pragma unroll
  for (int tt = 0; tt < LIN_TILES; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // K-steps in batches of LIN_U: a batch's loads (LIN_U x (LIN_TILES + 1) 16-byte
  // fragments) are all issued before its MFMAs, and the next batch is issued before
  // this one is consumed, so ~2 batches per wave are in flight (a plain loop makes the
  // compiler wait for each load before its MFMA).
  const int nk = H / 32;
  u32x4 wv[2][LIN_U], xv[2][LIN_U][LIN_TILES];
  auto load_batch = [&](int b, int kk) {
#pragma unroll
    for (int u = 0; u < LIN_U; ++u) {
      const int k = min(kk + u, nk - 1);
      wv[b][u] = *reinterpret_cast<const u32x4*>(wr + 32 * k);
#pragma unroll
      for (int tt = 0; tt < LIN_TILES; ++tt) xv[b][u][tt] = *reinterpret_cast<const u32x4*>(xr[tt] + 32 * k);
    }
  };
  auto mma_batch = [&](int b, int kk) {
#pragma unroll
    for (int u = 0; u < LIN_U; ++u) {
      if (kk + u < nk) {
        const u32x4 w = hv ? wv[b][u] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int tt = 0; tt < LIN_TILES; ++tt)
          acc[tt] = mfma16x16x32(as_bf16x8(xv[b][u][tt]), as_bf16x8(w), acc[tt]);
      }
    }
  };
  load_batch(0, 0);
  int kk = 0;
  for (; kk + LIN_U < nk; kk += 2 * LIN_U) {
    load_batch(1, kk + LIN_U);
    mma_batch(0, kk);
    if (kk + 2 * LIN_U < nk) load_batch(0, kk + 2 * LIN_U);
    mma_batch(1, kk + LIN_U);
  }
  if (kk < nk) mma_batch(0, kk);
  if (!hv) return;
  const float bb = bias ? bias[n] : 0.f;
#pragma unroll
  for (int tt = 0; tt < LIN_TILES; ++tt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t tok = tok0 + 16 * tt + 4 * j + i;
      if (tok < ntok) {
        const int b = static_cast<int>(tok / T), t = static_cast<int>(tok % T);
        scores[((int64_t)b * Hkv + n) * ld_s + t] = acc[tt][i] + bb;
      }
    }
  }
}

// ------------------------------------------------------------------ MLP bf16
constexpr int MLP_BM = 256;  // inner units per work-group
constexpr int MLP_BN = 256;  // tokens per work-group
constexpr int MLP_BK = 64;   // K per stage: 128-byte row segments, two MFMA K-steps
constexpr int MLP_THREADS = 512;                    // 8 waves: 4 (units) x 2 (tokens)
constexpr int MLP_ROWB = MLP_BK * 2;                // bytes per LDS row (128)
constexpr int MLP_TILEB = 256 * MLP_ROWB;           // 32 KB: one stage of one operand
constexpr int MLP_WSLOTS = 2;                       // W1 ring (L2-resident operand)
constexpr int MLP_XSLOTS = 3;                       // hidden-state ring (streamed from HBM)
constexpr int MLP_LDSB = (MLP_WSLOTS + MLP_XSLOTS) * MLP_TILEB;  // 160 KB: all of a CU's LDS

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// LDS row r holds the 64 K-values of one row as eight 16-byte chunks; chunk c is stored
// in slot c ^ (r & 7).  A ds_read_b128 is served eight lanes (128 bytes, all banks) at
// a time; the eight lanes of a fragment read read eight consecutive rows at one logical
// chunk, and the swizzle puts them in eight distinct 16-byte bank groups (conflict-free;
// measured on gfx950 as fast as a linear read).
__device__ __forceinline__ int swz_slot(int row, int chunk) { return chunk ^ (row & 7); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * MLP_ROWB + 16 * swz_slot(row, chunk); }

struct MlpArgs {
  const uint16_t* X;   // [ntok][H]
  const uint16_t* W1;  // [inner][H]
  const float* b1;     // [inner] or null
  const float* W2;     // [Hkv][inner]
  float* part;         // [inner/MLP_BM][ntok][16]
  int ntok, H, inner, Hkv;
};

__global__ __launch_bounds__(MLP_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void score_mlp_bf16_kernel(MlpArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[MLP_LDSB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, j = lane >> 4;
  const int wm = wid & 3, wn = wid >> 2;  // wave tile: inner [64wm,+64) x tokens [128wn,+128)
  // XCD-aware order: work-groups are dispatched round-robin over the 8 XCDs, so the
  // nparts slices of one token tile get ids b, b+8, ... (same XCD, adjacent in time)
  // and share that tile's hidden states through the XCD's L2.
  const int nparts = a.inner / MLP_BM;
  const int grp = blockIdx.x / (8 * nparts), r8 = blockIdx.x % (8 * nparts);
  const int64_t tile = (int64_t)grp * 8 + (r8 % 8);
  const int part = r8 / 8;
  const int64_t tok0 = tile * MLP_BN;
  if (tok0 >= a.ntok) return;
  const int in0 = part * MLP_BM;
  const int H = a.H;

  // Direct global->LDS copies: one global_load_lds_dwordx4 writes a wave's 64 lanes x
  // 16 B to 1 KB of contiguous LDS (lane i at +16 i), i.e. 8 rows of a stage.  A stage
  // of either operand is 32 such blocks; wave w fills blocks 4w .. 4w+3 of both.  Lane i
  // covers row 8 blk + i/8, slot i%8, and fetches the chunk the swizzle maps to that
  // slot, so each instruction reads eight whole 128-byte row segments.
  // Copies go through buffer resources based at this tile's first row: a per-lane 32-bit
  // offset in one VGPR plus a uniform offset (block, K-step) in an SGPR, so the
  // 128-entry accumulator still fits in 256 VGPRs.  Every address is in bounds by
  // construction (tail rows are clamped), the resource range is only a backstop.  Row
  // 8 blk + i/8 has row & 7 == i/8 for every block, so the swizzled chunk is the same
  // for all of a wave's blocks.
  const int chunk = swz_slot(lane >> 3, lane & 7);  // the swizzle is an involution
  const int rowb = 2 * H;                            // bytes per row
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.W1 + (int64_t)in0 * H), (short)0, MLP_BM * rowb, 0x00020000);
  const int64_t xrows = min((int64_t)MLP_BN, (int64_t)a.ntok - tok0);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.X + tok0 * H), (short)0, (int)(xrows * rowb), 0x00020000);
  const uint32_t woff = (uint32_t)((lane >> 3) * rowb + 16 * chunk);
  uint32_t xoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = min(8 * (4 * wid + q) + (lane >> 3), (int)xrows - 1);  // tail: duplicate rows, results dropped
    xoff[q] = (uint32_t)(row * rowb + 16 * chunk);
  }
  uint8_t* const wring = lds;
  uint8_t* const xring = lds + MLP_WSLOTS * MLP_TILEB;
  auto issue_w1 = [&](int kt, int slot, int q) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t*)(wring + slot * MLP_TILEB + (4 * wid + q) * 1024),
                                             16, woff, (8 * (4 * wid + q)) * rowb + kt * MLP_ROWB, 0, 0);
  };
  auto issue_x1 = [&](int kt, int slot, int q) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void_t*)(xring + slot * MLP_TILEB + (4 * wid + q) * 1024),
                                             16, xoff[q], kt * MLP_ROWB, 0, 0);
  };
  auto issue_w = [&](int kt, int slot) {
    uint8_t* st = wring + slot * MLP_TILEB + 4 * wid * 1024;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t*)(st + q * 1024), 16, woff,
                                               (8 * (4 * wid + q)) * rowb + kt * MLP_ROWB, 0, 0);
  };
  auto issue_x = [&](int kt, int slot) {
    uint8_t* st = xring + slot * MLP_TILEB + 4 * wid * 1024;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void_t*)(st + q * 1024), 16, xoff[q],
                                               kt * MLP_ROWB, 0, 0);
  };
  // fragment of K-step ks (0/1) of the stage in slot kt % ring: 16 rows x 32 K, lane
  // (n, j) holds row n, logical chunk 4 ks + j (eight consecutive K-values)
  auto lds_a = [&](int kt, int ks, int mt) {
    const uint8_t* s = wring + (kt % MLP_WSLOTS) * MLP_TILEB;
    return as_bf16x8(*reinterpret_cast<const u32x4*>(s + swz(64 * wm + 16 * mt + n, 4 * ks + j)));
  };
  auto lds_b = [&](int kt, int ks, int nt) {
    const uint8_t* s = xring + (kt % MLP_XSLOTS) * MLP_TILEB;
    return as_bf16x8(*reinterpret_cast<const u32x4*>(s + swz(128 * wn + 16 * nt + n, 4 * ks + j)));
  };
  // a plain barrier after this wave's LDS reads: __syncthreads() would also wait for
  // every copy still in flight
  auto barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) (vmcnt/expcnt max)
    __builtin_amdgcn_s_barrier();
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = H / MLP_BK;
  // Pipeline.  Stage s of W1 lives in W slot s % 2, stage s of the hidden states in X
  // slot s % 3.  Step kt runs the MFMAs of stage kt in two K-steps; fragments are read
  // one K-step ahead (A into a second register set, B refilled in place right after its
  // last use).  Half-way through step kt, after the MFMAs of K-step 0 are issued:
  //   1. wait for this wave's copies of W1 stage kt+1 and X stage kt+1 (X stage kt+2
  //      may still fly)
  //   2. barrier: stage kt+1 is complete for every wave, and every wave has read all of
  //      stage kt into registers (its K-step 1 fragments were read during K-step 0), so
  //      both of stage kt's slots are free
  //   3. copy W1 stage kt+2 into W slot kt % 2, X stage kt+3 into X slot kt % 3, one
  //      copy per MFMA column of K-step 1 so the matrix pipe never waits on the issue
  // W1 (4 MB, shared by every work-group, L2-resident) gets one step to arrive, the
  // hidden states (HBM) two.  Copies past the last stage are clamped to it (same bytes,
  // still into the free slot) so every step issues the same instructions and the wait
  // counts stay exact; the fragments read in the last step (for a stage nk that does
  // not exist) come from a slot whose copy has landed and that no copy targets, and are
  // never used.  sched_barrier(0) pins the order against the instruction scheduler.
  // prologue: [W0 X0] [X1] [W1 X2]
  issue_w(0, 0);
  issue_x(0, 0);
  issue_x(min(1, nk - 1), 1);
  issue_w(min(1, nk - 1), 1);
  issue_x(min(2, nk - 1), 2);
  __builtin_amdgcn_s_waitcnt(0x0F7C);  // vmcnt(12): W0, X0 landed (expcnt/lgkmcnt max)
  barrier();
  bf16x8 fa0[4], fa1[4], fb[8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) fa0[mt] = lds_a(0, 0, mt);
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) fb[nt] = lds_b(0, 0, nt);

  // The next A fragments are read after the first column of MFMAs, when the oldest B
  // reads have returned, so at most 12 LDS reads are ever outstanding.  The loop is
  // rotated so that its back edge sits at the mid-step barrier, which waits for every
  // LDS read anyway: the compiler's conservative wait at a loop header costs nothing
  // there, and inside the body it waits only for the fragment the next MFMA needs.
  auto kstep0 = [&](int kt) {  // K-step 0 of stage kt; reads K-step 1 of stage kt
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma16x16x32(fa0[mt], fb[nt], acc[mt][nt]);
      if (nt == 0) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) fa1[mt] = lds_a(kt, 1, mt);
      }
      fb[nt] = lds_b(kt, 1, nt);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // K-step 1 of stage kt; reads K-step 0 of kt+1 and spreads the copies of W1 stage
  // kt+2 and X stage kt+3 over its MFMA columns (all W1 copies before all X copies, so
  // the in-order vmcnt waits above stay exact)
  auto kstep1 = [&](int kt, bool next) {
    const int ws = kt % MLP_WSLOTS, xs = kt % MLP_XSLOTS;
    const int wk = min(kt + 2, nk - 1), xk = min(kt + 3, nk - 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma16x16x32(fa1[mt], fb[nt], acc[mt][nt]);
      if (next) {
        if (nt < 4) issue_w1(wk, ws, nt);
        else issue_x1(xk, xs, nt - 4);
        if (nt == 0) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) fa0[mt] = lds_a(kt + 1, 0, mt);
        }
        fb[nt] = lds_b(kt + 1, 0, nt);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto mid = [&]() {  // stage kt+1 ready; stage kt's slots free for the copies above
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F74);  // vmcnt(4): only X stage kt+2 may still fly
    barrier();
  };
  kstep0(0);
  for (int kt = 0; kt + 1 < nk; ++kt) {
    mid();
    kstep1(kt, true);
    kstep0(kt + 1);
  }
  kstep1(nk - 1, false);
  // the clamped copies of the last steps are still in flight: drain them before the
  // epilogue reuses LDS
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- epilogue: u = GELU(acc + b1) (fp32), s_part = W2[:, slice] . u on MFMA
  // acc[mt][nt][i] = A^T[inner 64wm + 16mt + 4j + i][token 128wn + 16nt + n]
  // second-layer K-step kst uses M-tiles 2kst, 2kst+1; K-slot v of lane group j is
  // inner row 32kst + 4j + v (v < 4) or 32kst + 16 + 4j + (v - 4) (v >= 4).
  u32x4 w2hi[2], w2lo[2];
#pragma unroll
  for (int kst = 0; kst < 2; ++kst) {
    float wv[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const int r = 64 * wm + 32 * kst + (v < 4 ? 4 * j + v : 16 + 4 * j + (v - 4));
      wv[v] = (n < a.Hkv) ? a.W2[(int64_t)n * a.inner + in0 + r] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x2 hl = split_bf16x2(wv[2 * q], wv[2 * q + 1]);
      w2hi[kst][q] = hl[0];
      w2lo[kst][q] = hl[1];
    }
  }
  float b1v[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = in0 + 64 * wm + 16 * mt + 4 * j + i;
      b1v[mt][i] = a.b1 ? a.b1[r] : 0.f;
    }
  f32x4 sacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kst = 0; kst < 2; ++kst) {
      float u[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u[i] = gelu_erf(acc[2 * kst][nt][i] + b1v[2 * kst][i]);
        u[i + 4] = gelu_erf(acc[2 * kst + 1][nt][i] + b1v[2 * kst + 1][i]);
      }
      u32x4 uhi, ulo;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 hl = split_bf16x2(u[2 * q], u[2 * q + 1]);
        uhi[q] = hl[0];
        ulo[q] = hl[1];
      }
      sacc[nt] = mfma16x16x32(as_bf16x8(w2hi[kst]), as_bf16x8(uhi), sacc[nt]);
      sacc[nt] = mfma16x16x32(as_bf16x8(w2lo[kst]), as_bf16x8(uhi), sacc[nt]);
      sacc[nt] = mfma16x16x32(as_bf16x8(w2hi[kst]), as_bf16x8(ulo), sacc[nt]);
    }
  }
  // sacc[nt][i] = partial s[head 4j+i][token 128wn + 16nt + n] over this wave's 64 units
  __syncthreads();  // done with the GEMM tiles; reuse LDS for the cross-wave sum
  float* red = reinterpret_cast<float*>(lds);  // [4 wm][256 tokens][16 heads]
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      red[(wm * MLP_BN + 128 * wn + 16 * nt + n) * 16 + 4 * j + i] = sacc[nt][i];
  __syncthreads();
  float* dst = a.part + ((int64_t)part * a.ntok) * 16;
  for (int e = tid; e < MLP_BN * 16; e += MLP_THREADS) {
    const int t = e >> 4, h = e & 15;
    const int64_t tok = tok0 + t;
    if (tok < a.ntok && h < a.Hkv) {
      float sum = red[(0 * MLP_BN + t) * 16 + h];
      sum += red[(1 * MLP_BN + t) * 16 + h];
      sum += red[(2 * MLP_BN + t) * 16 + h];
      sum += red[(3 * MLP_BN + t) * 16 + h];
      dst[tok * 16 + h] = sum;
    }
  }
}

// One thread per token: the token's 16-float partial rows are contiguous (four 16-byte
// loads per part), and for each head consecutive threads store consecutive positions.
__global__ __launch_bounds__(256) void score_mlp_finish_kernel(const float* __restrict__ part,
                                                               int nparts, int ntok, int Hkv,
                                                               const float* __restrict__ b2, int T,
                                                               float* __restrict__ scores,
                                                               int64_t ld_s) {
  const int64_t tok = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tok >= ntok) return;
  f32x4 s[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) s[c] = reinterpret_cast<const f32x4*>(part + tok * 16)[c];
  for (int q = 1; q < nparts; ++q) {
    const f32x4* pq = reinterpret_cast<const f32x4*>(part + ((int64_t)q * ntok + tok) * 16);
#pragma unroll
    for (int c = 0; c < 4; ++c) s[c] += pq[c];
  }
  const int b = static_cast<int>(tok / T), t = static_cast<int>(tok % T);
  float* dst = scores + (int64_t)b * Hkv * ld_s + t;
#pragma unroll
  for (int h = 0; h < 16; ++h)
    if (h < Hkv) dst[(int64_t)h * ld_s] = s[h >> 2][h & 3] + (b2 ? b2[h] : 0.f);
}

// ------------------------------------------------------------------ small batches
// Decode steps score only a handful of tokens (one per sequence): the first layer is
// split over K (small_gemm.h), one slice per wave.
template <int NTT>
__global__ __launch_bounds__(256) void score_small_gemm_kernel(SmallGemm g) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= g.rtiles * g.ksplit) return;
  small_gemm_slice<NTT>(g, w);
}

// K slices are summed in a fixed order; loads of absent slices (ks >= ksplit) read the
// last slice and contribute an exact zero, so every load is unconditional.
constexpr int SMALL_MAX_KSPLIT = 32;  // hidden size <= 8192

// MLP epilogue: one work-group per token, one thread per inner unit (inner <= 1024).
__global__ __launch_bounds__(1024) void score_small_mlp_epi_kernel(
    const float* __restrict__ part, int ksplit, int ntok, int inner, const float* __restrict__ b1,
    const float* __restrict__ W2, const float* __restrict__ b2, int Hkv, int T,
    float* __restrict__ scores, int64_t ld_s) {
  __shared__ float red[16][16];
  const int tok = blockIdx.x, u = threadIdx.x;
  const int lane = u & 63, wid = u >> 6;
  float pv[SMALL_MAX_KSPLIT];
#pragma unroll
  for (int ks = 0; ks < SMALL_MAX_KSPLIT; ++ks)
    pv[ks] = part[((int64_t)min(ks, ksplit - 1) * ntok + tok) * inner + u];
  float w2v[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) w2v[h] = W2[(int64_t)min(h, Hkv - 1) * inner + u];
  const float bias1 = b1 ? b1[u] : 0.f;
  float a = 0.f;
#pragma unroll
  for (int ks = 0; ks < SMALL_MAX_KSPLIT; ++ks) a += (ks < ksplit) ? pv[ks] : 0.f;
  a += bias1;
  const float g = gelu_erf(a);
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    if (h < Hkv) {
      const float v = wave_sum(g * w2v[h]);
      if (lane == 0) red[h][wid] = v;
    }
  }
  __syncthreads();
  if (u < Hkv) {
    float sacc = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) sacc += red[u][w];
    if (b2) sacc += b2[u];
    const int b = tok / T, t = tok % T;
    scores[((int64_t)b * Hkv + u) * ld_s + t] = sacc;
  }
}

// Linear epilogue: sum the K slices of each (token, head) and add the bias.
__global__ __launch_bounds__(256) void score_small_linear_epi_kernel(
    const float* __restrict__ part, int ksplit, int ntok, int Hkv, const float* __restrict__ bias,
    int T, float* __restrict__ scores, int64_t ld_s) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= ntok * Hkv) return;
  const int tok = idx / Hkv, h = idx % Hkv;
  float pv[SMALL_MAX_KSPLIT];
#pragma unroll
  for (int ks = 0; ks < SMALL_MAX_KSPLIT; ++ks) pv[ks] = part[((int64_t)min(ks, ksplit - 1) * ntok + tok) * 16 + h];
  float a = 0.f;
#pragma unroll
  for (int ks = 0; ks < SMALL_MAX_KSPLIT; ++ks) a += (ks < ksplit) ? pv[ks] : 0.f;
  if (bias) a += bias[h];
  const int b = tok / T, t = tok % T;
  scores[((int64_t)b * Hkv + h) * ld_s + t] = a;
}

}  // namespace kvp

using namespace kvp;

static bool small_path(const kvp_scorer* sc, int64_t ntok) {
  return sc->wdtype == KVP_BF16 && ntok <= SMALL_MAX_TOK && sc->hidden % SMALL_KSLICE == 0 &&
         sc->hidden / SMALL_KSLICE <= SMALL_MAX_KSPLIT &&
         (sc->kind == KVP_SCORER_LINEAR || sc->inner <= 1024);
}

extern "C" size_t kvp_score_workspace_size(const kvp_scorer* sc, int32_t B, int32_t T) {
  if (!sc || B <= 0 || T <= 0) return 0;
  const int64_t ntok = (int64_t)B * T;
  if (sc->kind == KVP_SCORER_MLP && (sc->inner <= 0 || sc->inner % MLP_BM != 0)) return 0;
  if (small_path(sc, ntok)) {
    const int rows = sc->kind == KVP_SCORER_MLP ? sc->inner : 16;
    return (size_t)(sc->hidden / SMALL_KSLICE) * ntok * cdiv(rows, 16) * 16 * sizeof(float);
  }
  if (sc->kind != KVP_SCORER_MLP) return 0;
  return (size_t)(sc->inner / MLP_BM) * (size_t)ntok * 16 * sizeof(float);
}

// The split-K partial sums of a small batch's first layer, alone (the MLP decode step
// finishes them inside the delayed-step kernel): part[ks][token][unit], ks < H / 256.
bool kvp_score_small_mlp_ok(const kvp_scorer* sc, int ntok) {
  return sc->kind == KVP_SCORER_MLP && small_path(sc, ntok) && sc->inner % 256 == 0;
}

SmallGemm kvp::small_gemm_of(const kvp_scorer* sc, const void* hidden, int ntok, int rows, float* part) {
  SmallGemm g;
  g.x = reinterpret_cast<const uint16_t*>(hidden);
  g.w = reinterpret_cast<const uint16_t*>(sc->w1);
  g.part = part;
  g.rows = rows;
  g.ntok = ntok;
  g.H = sc->hidden;
  g.rtiles = cdiv(rows, 16);
  g.ksplit = sc->hidden / SMALL_KSLICE;
  return g;
}

static void launch_small_gemm(const SmallGemm& g, hipStream_t stream) {
  const dim3 grid(cdiv(g.rtiles * g.ksplit, 4)), b(256);
  switch (cdiv(g.ntok, 16)) {
    case 1: hipLaunchKernelGGL(score_small_gemm_kernel<1>, grid, b, 0, stream, g); break;
    case 2: hipLaunchKernelGGL(score_small_gemm_kernel<2>, grid, b, 0, stream, g); break;
    case 3: hipLaunchKernelGGL(score_small_gemm_kernel<3>, grid, b, 0, stream, g); break;
    default: hipLaunchKernelGGL(score_small_gemm_kernel<4>, grid, b, 0, stream, g); break;
  }
}

kvp_status kvp_launch_score_small_partials(const kvp_scorer* sc, const void* hidden, int ntok,
                                           float* part, hipStream_t stream) {
  launch_small_gemm(small_gemm_of(sc, hidden, ntok, sc->inner, part), stream);
  KVP_LAUNCH_CHECK();
  return KVP_OK;
}

kvp_status kvp_launch_score(const kvp_scorer* sc, const void* hidden, int B, int T, float* scores,
                            int64_t ld_s, void* ws, hipStream_t stream) {
  const int ntok = B * T;
  const int H = sc->hidden, Hkv = sc->n_kv_heads;
  if (small_path(sc, ntok)) {
    const int ksplit = H / SMALL_KSLICE;
    const bool mlp = sc->kind == KVP_SCORER_MLP;
    float* part = reinterpret_cast<float*>(ws);
    launch_small_gemm(small_gemm_of(sc, hidden, ntok, mlp ? sc->inner : Hkv, part), stream);
    KVP_LAUNCH_CHECK();
    if (mlp) {
      hipLaunchKernelGGL(score_small_mlp_epi_kernel, dim3(ntok), dim3(sc->inner), 0, stream, part, ksplit,
                         ntok, sc->inner, sc->b1, sc->w2, sc->b2, Hkv, T, scores, ld_s);
    } else {
      hipLaunchKernelGGL(score_small_linear_epi_kernel, dim3(cdiv(ntok * Hkv, 256)), dim3(256), 0, stream,
                         part, ksplit, ntok, Hkv, sc->b1, T, scores, ld_s);
    }
    KVP_LAUNCH_CHECK();
    return KVP_OK;
  }
  if (sc->kind == KVP_SCORER_LINEAR) {
    if (sc->wdtype == KVP_F32) {
      const int64_t n = (int64_t)ntok * Hkv;
      hipLaunchKernelGGL(score_linear_f32_kernel, dim3((unsigned)cdiv64(n, 256)), dim3(256), 0, stream,
                         reinterpret_cast<const float*>(hidden), reinterpret_cast<const float*>(sc->w1),
                         sc->b1, ntok, H, Hkv, T, scores, ld_s);
    } else {
      const int64_t waves = cdiv64(ntok, 16 * LIN_TILES);
      hipLaunchKernelGGL(score_linear_bf16_kernel, dim3((unsigned)cdiv64(waves, 4)), dim3(256), 0, stream,
                         reinterpret_cast<const uint16_t*>(hidden),
                         reinterpret_cast<const uint16_t*>(sc->w1), sc->b1, ntok, H, Hkv, T, scores, ld_s);
    }
    KVP_LAUNCH_CHECK();
    return KVP_OK;
  }
  MlpArgs m;
  m.X = reinterpret_cast<const uint16_t*>(hidden);
  m.W1 = reinterpret_cast<const uint16_t*>(sc->w1);
  m.b1 = sc->b1;
  m.W2 = sc->w2;
  m.part = reinterpret_cast<float*>(ws);
  m.ntok = ntok;
  m.H = H;
  m.inner = sc->inner;
  m.Hkv = Hkv;
  const int nparts = sc->inner / MLP_BM;
  const int64_t tiles = cdiv64(ntok, MLP_BN);
  hipLaunchKernelGGL(score_mlp_bf16_kernel, dim3((unsigned)(cdiv64(tiles, 8) * 8 * nparts)),
                     dim3(MLP_THREADS), 0, stream, m);
  KVP_LAUNCH_CHECK();
  hipLaunchKernelGGL(score_mlp_finish_kernel, dim3((unsigned)cdiv64(ntok, 256)), dim3(256), 0, stream, m.part,
                     nparts, ntok, Hkv, sc->b2, T, scores, ld_s);
  KVP_LAUNCH_CHECK();
  return KVP_OK;
}
