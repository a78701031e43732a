// The delayed-eviction step of one pair, shared by the step kernel and by the fused
// decode step (whose merge kernel applies it after the attention has read the ring).
//
// Method: DMS article (euno.news), "Delayed Eviction" -- a token flagged for eviction
// is not removed at once but kept in a short buffer for a fixed number of steps and
// deleted when that window expires; "How DMS works" step 3 -- the keep/evict signal
// is binary per token.  KVzap digest (max5.ai), practical application -- the most
// recent tokens are always kept and low-scoring ones are removed.  BeaconKV briefing
// (jiinsi.com), body -- with a low-precision pool the token is demoted instead.
#pragma once

#include "kvp_internal.h"

namespace kvp {


struct StepArgs {
  kvp_paged_kv kv;
  kvp_ring ring;
  const void* k_new;
  const void* v_new;
  const float* s_new;
  int64_t ld_s;
  float tau;
  const float* tau_dev;  // if set, tau is read from here
  int p;
  int* pos_dev;  // if set: [position, arrivals]; the position is read from here and advanced
  // Fused linear scorer (s_new unused when x_new is set): the new token's score of pair
  // (b, h) is x_new[b] . w[h] + bias[h], computed by the pair's wave.
  const void* x_new;  // [B][H] hidden states of the new tokens
  const void* w;      // [Hkv][H] scorer weights (nn.Linear layout), same dtype as x_new
  const float* bias;  // [Hkv] or null
  float* s_out;       // [B * Hkv] or null: the scores, as stored in the ring
  int H, Hkv, x_bf16;
  // Fused MLP finish (s_new unused when part is set): part[ks][b][unit] holds the split-K
  // partial sums of the first layer for the new token of sequence b (ks < ksplit); the
  // pair's wave adds them, then b1, GELU, the row h of W2 and b2.
  const float* part;
  int ksplit, ntok, inner;
  const float* b1;
  const float* w2;  // [Hkv][inner]
  const float* b2;  // [Hkv] or null
};

template <typename E>
__device__ __forceinline__ float to_f32(E x);
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }

// One lane's share of x . w over H elements (16-byte loads, fp32 fused multiply-adds in
// a fixed order), summed across the wave.  Eight 16-byte pieces of x and of w per lane
// are requested together (addresses clamped in bounds, pieces past the end zeroed), so
// H = 4096 in bf16 costs one memory round trip.
template <typename X>
__device__ __forceinline__ float wave_dot(const X* __restrict__ x, const X* __restrict__ w, int H) {
  constexpr int V = 16 / sizeof(X);
  constexpr int NB = 8;
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  for (int i0 = lane * V; i0 < H; i0 += 64 * V * NB) {
    u32x4 xv[NB], wv[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int i = min(i0 + 64 * V * k, H - V);
      xv[k] = *reinterpret_cast<const u32x4*>(x + i);
      wv[k] = *reinterpret_cast<const u32x4*>(w + i);
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      if (i0 + 64 * V * k >= H) {  // a clamped repeat: contributes exactly 0
        xv[k] = u32x4{0u, 0u, 0u, 0u};
        wv[k] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (sizeof(X) == 2) {
          acc = fmaf(bf16_to_f32(xv[k][e] & 0xffffu), bf16_to_f32(wv[k][e] & 0xffffu), acc);
          acc = fmaf(bf16_to_f32(xv[k][e] >> 16), bf16_to_f32(wv[k][e] >> 16), acc);
        } else {
          acc = fmaf(__uint_as_float(xv[k][e]), __uint_as_float(wv[k][e]), acc);
        }
      }
    }
  }
  return wave_sum(acc);
}

// MLP score of one new token by one wave: lane l owns units 256c + 4l .. 256c + 4l + 3
// (NC = inner / 256); the K slices are summed in slice order, KB slices' loads at a time
// (at most 32 16-byte loads in flight per lane, so the caller keeps its occupancy).
template <int NC>
__device__ __forceinline__ float wave_mlp_finish(const StepArgs& a, int tok, int h) {
  const int lane = threadIdx.x & 63;
  f32x4 acc[NC], b1v[NC], w2v[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int u = 256 * c + 4 * lane;
    acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    b1v[c] = a.b1 ? *reinterpret_cast<const f32x4*>(a.b1 + u) : f32x4{0.f, 0.f, 0.f, 0.f};
    w2v[c] = *reinterpret_cast<const f32x4*>(a.w2 + (int64_t)h * a.inner + u);
  }
  constexpr int KB = NC <= 2 ? 16 : 8;
  for (int ks0 = 0; ks0 < a.ksplit; ks0 += KB) {
    f32x4 v[KB][NC];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int ks = min(ks0 + k, a.ksplit - 1);  // in bounds; slices past the end add 0
#pragma unroll
      for (int c = 0; c < NC; ++c)
        v[k][c] = *reinterpret_cast<const f32x4*>(a.part + ((int64_t)ks * a.ntok + tok) * a.inner +
                                                  256 * c + 4 * lane);
    }
#pragma unroll
    for (int k = 0; k < KB; ++k)
      if (ks0 + k < a.ksplit) {
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] += v[k][c];
      }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) s = fmaf(gelu_erf(acc[c][e] + b1v[c][e]), w2v[c][e], s);
  s = wave_sum(s);
  if (a.b2) s += a.b2[h];
  return s;
}


// Appending position p to `pair` (one wave): the token at p - window leaves ring slot
// p mod window and is appended to the pool iff its score >= tau (else dropped, or
// demoted to the low-precision pool when there is one); the new token enters the slot
// with its score (given, or computed by the fused scorer).  The pool length and the
// tau value are requested before the position is needed, the block-table entry of the
// append with the ring slot, so the common path costs two memory round trips.
template <typename E, int D>
__device__ __forceinline__ void step_pair(const StepArgs& a, int pair, int p) {
  const int lane = threadIdx.x & 63;
  // independent of the position: requested first
  const int len = a.kv.length[pair];
  const int len8 = a.kv.num_pages8 > 0 ? a.kv.length8[pair] : 0;
  const float tau = a.tau_dev ? a.tau_dev[0] : a.tau;
  const float s_given = (!a.x_new && !a.part) ? a.s_new[(int64_t)pair * a.ld_s] : 0.f;
  constexpr int PER = (D + 63) / 64;
  E kn[PER], vn[PER];  // the new token
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int dd = min(lane + 64 * e, D - 1);
    kn[e] = reinterpret_cast<const E*>(a.k_new)[(int64_t)pair * D + dd];
    vn[e] = reinterpret_cast<const E*>(a.v_new)[(int64_t)pair * D + dd];
  }
  const int w = a.ring.window;
  const int slot = ((p % w) + w) % w;  // a negative position (a caller's bug) stays in bounds
  const int rp = slot / PAGE, rs = slot % PAGE;
  const int64_t roff = ((int64_t)pair * (w / PAGE) + rp) * PAGE * D;
  E* rk = reinterpret_cast<E*>(a.ring.k) + roff + rs * D;  // K row of the slot
  E* rv = reinterpret_cast<E*>(a.ring.v) + roff + rs;      // V column, stride PAGE
  const int old_pos = a.ring.pos[(int64_t)pair * w + slot];
  const float old_s = a.ring.score[(int64_t)pair * w + slot];
  E ko[PER], vo[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int dd = lane + 64 * e;
    if (dd < D) {
      ko[e] = rk[dd];
      vo[e] = rv[dd * PAGE];
    }
  }
  // block-table entries an append would write into (the last, partly filled page),
  // requested with the ring slot whether or not the token is retained
  const int j = len / PAGE, sl = len % PAGE;
  const int bt_last = (sl != 0 && j < a.kv.max_pages_per_pair)
                          ? a.kv.block_table[(int64_t)pair * a.kv.max_pages_per_pair + j] : -1;
  const int j8 = len8 / PAGE, sl8 = len8 % PAGE;
  const int bt8_last = (a.kv.num_pages8 > 0 && sl8 != 0 && j8 < a.kv.max_pages8_per_pair)
                           ? a.kv.block_table8[(int64_t)pair * a.kv.max_pages8_per_pair + j8] : -1;
  // the new token's score (fused scorer): needed only at the end, requested after the
  // ring loads so both latencies overlap
  float s_new = 0.f;
  if (a.x_new) {
    const int b = pair / a.Hkv, h = pair % a.Hkv;
    if (a.x_bf16)
      s_new = wave_dot(reinterpret_cast<const uint16_t*>(a.x_new) + (int64_t)b * a.H,
                       reinterpret_cast<const uint16_t*>(a.w) + (int64_t)h * a.H, a.H);
    else
      s_new = wave_dot(reinterpret_cast<const float*>(a.x_new) + (int64_t)b * a.H,
                       reinterpret_cast<const float*>(a.w) + (int64_t)h * a.H, a.H);
    if (a.bias) s_new += a.bias[h];
  } else if (a.part) {
    const int b = pair / a.Hkv, h = pair % a.Hkv;
    switch (a.inner >> 8) {
      case 1: s_new = wave_mlp_finish<1>(a, b, h); break;
      case 2: s_new = wave_mlp_finish<2>(a, b, h); break;
      case 3: s_new = wave_mlp_finish<3>(a, b, h); break;
      default: s_new = wave_mlp_finish<4>(a, b, h); break;
    }
  }
  if (old_pos >= 0) {
    if (old_s >= tau) {
      // retain: append to the pool (allocating a page when the last one is full)
      int pg = -1;
      if (sl == 0) {
        if (j >= a.kv.max_pages_per_pair) {
          if (lane == 0) atomicOr(a.kv.err, KVP_ERR_TABLE_FULL);
        } else {
          int got = 0;
          if (lane == 0) got = atomicAdd(a.kv.page_top, 1);
          got = __shfl(got, 0);
          if (got >= a.kv.num_pages) {
            if (lane == 0) atomicOr(a.kv.err, KVP_ERR_POOL_FULL);
          } else {
            pg = got;
            if (lane == 0) a.kv.block_table[(int64_t)pair * a.kv.max_pages_per_pair + j] = pg;
          }
        }
      } else {
        pg = bt_last;
      }
      if (pg >= 0) {
        E* kp = reinterpret_cast<E*>(a.kv.k_pages) + (int64_t)pg * PAGE * D + sl * D;
        E* vp = reinterpret_cast<E*>(a.kv.v_pages) + (int64_t)pg * PAGE * D + sl;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int dd = lane + 64 * e;
          if (dd < D) {
            kp[dd] = ko[e];
            vp[dd * PAGE] = vo[e];
          }
        }
        if (lane == 0) {
          a.kv.page_pos[(int64_t)pg * PAGE + sl] = old_pos;
          a.kv.length[pair] = len + 1;
        }
      }
    } else if (a.kv.num_pages8 > 0) {
      // demote to the low-precision pool (BeaconKV): absmax per row, K and V separately;
      // int8, int4 or fp8 E4M3 codes
      float kf[PER], vf[PER];
      float ka = 0.f, va = 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int dd = lane + 64 * e;
        kf[e] = (dd < D) ? to_f32<E>(ko[e]) : 0.f;
        vf[e] = (dd < D) ? to_f32<E>(vo[e]) : 0.f;
        ka = fmaxf(ka, fabsf(kf[e]));
        va = fmaxf(va, fabsf(vf[e]));
      }
      ka = wave_max(ka);
      va = wave_max(va);
      const bool i4 = lp_bits_of(a.kv) == 4, f8 = lp_is_fp8(a.kv);
      const float qmax = f8 ? 448.0f : (i4 ? 7.0f : 127.0f);
      const float ks = ka / qmax, vs = va / qmax;
      const int j = j8, sl = sl8;
      int pg = -1;
      if (sl == 0) {
        if (j >= a.kv.max_pages8_per_pair) {
          if (lane == 0) atomicOr(a.kv.err, KVP_ERR_POOL8_FULL);
        } else {
          int got = 0;
          if (lane == 0) got = atomicAdd(a.kv.page8_top, 1);
          got = __shfl(got, 0);
          if (got >= a.kv.num_pages8) {
            if (lane == 0) atomicOr(a.kv.err, KVP_ERR_POOL8_FULL);
          } else {
            pg = got;
            if (lane == 0) a.kv.block_table8[(int64_t)pair * a.kv.max_pages8_per_pair + j] = pg;
          }
        }
      } else {
        pg = bt8_last;
      }
      if (pg >= 0 && i4) {
        // int4: K row of d/2 bytes (dims 2i, 2i+1 share byte i: even lanes write, the odd
        // neighbour's code comes by shuffle); V^T rows of 8 bytes, this slot's nibble
        // merged into the byte it shares with slot sl ^ 1 (written at another step)
        int8_t* kp = a.kv.k8_pages + (int64_t)pg * PAGE * D / 2 + sl * (D / 2);
        uint8_t* vp = reinterpret_cast<uint8_t*>(a.kv.v8_pages) + (int64_t)pg * PAGE * D / 2 + sl / 2;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int dd = lane + 64 * e;
          const int kc = quant_code(kf[e], ks, qmax);
          const int kc1 = __shfl_down(kc, 1);
          if (dd < D) {
            if ((dd & 1) == 0) kp[dd / 2] = static_cast<int8_t>((kc & 0xf) | (kc1 << 4));
            const uint32_t vc = static_cast<uint32_t>(quant_code(vf[e], vs, qmax)) & 0xfu;
            uint8_t* vb = vp + dd * (PAGE / 2);
            const uint32_t old_b = *vb;
            *vb = static_cast<uint8_t>((sl & 1) ? ((old_b & 0x0fu) | (vc << 4)) : ((old_b & 0xf0u) | vc));
          }
        }
      } else if (pg >= 0) {
        int8_t* kp = a.kv.k8_pages + (int64_t)pg * PAGE * D + sl * D;
        int8_t* vp = a.kv.v8_pages + (int64_t)pg * PAGE * D + sl;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int dd = lane + 64 * e;
          if (dd < D) {
            kp[dd] = static_cast<int8_t>(f8 ? fp8_quant_code(kf[e], ks) : quant_code(kf[e], ks));
            vp[dd * PAGE] = static_cast<int8_t>(f8 ? fp8_quant_code(vf[e], vs) : quant_code(vf[e], vs));
          }
        }
      }
      if (pg >= 0) {
        if (lane == 0) {
          a.kv.k8_scale[(int64_t)pg * PAGE + sl] = ks;
          a.kv.v8_scale[(int64_t)pg * PAGE + sl] = vs;
          a.kv.page8_pos[(int64_t)pg * PAGE + sl] = old_pos;
          a.kv.length8[pair] = len8 + 1;
        }
      }
    }
  }
  // the new token enters the slot
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int dd = lane + 64 * e;
    if (dd < D) {
      rk[dd] = kn[e];
      rv[dd * PAGE] = vn[e];
    }
  }
  if (lane == 0) {
    a.ring.pos[(int64_t)pair * w + slot] = p;
    if (!a.x_new && !a.part) s_new = s_given;
    a.ring.score[(int64_t)pair * w + slot] = s_new;
    if (a.s_out) a.s_out[pair] = s_new;
  }
}

// Host: the step's kernel arguments (sc == nullptr: scores from s_new; a linear scorer
// reads x_new; an MLP scorer reads the split-K partial sums in part).
StepArgs make_step_args(const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                        const void* v_new, const float* s_new, int64_t ld_s, float tau,
                        const float* tau_dev, int p, int* pos_dev, const kvp_scorer* sc,
                        const void* x_new, float* s_out, const float* part);

}  // namespace kvp
