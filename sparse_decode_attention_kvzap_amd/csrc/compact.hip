// Compaction of the kept entries into the paged cache (gfx950).
//
// Method: DeInfer summary (gist.science, arXiv 2604.17709), method part (b) -- a
// preparation pass builds a remapping index list, then a copy pass moves the blocks
// into a compact, fixed-address KV buffer.  Here the index list is kvp_select's
// ordered kept_idx, the preparation pass is compact_plan_kernel (page counts, page
// bases by exclusive scan, lengths, capacity checks) and the copy pass is
// compact_copy_kernel.  KVzap practical application: only kept entries (plus the
// recent window) remain.  BeaconKV body: in DEMOTE_INT8 mode the other entries are
// kept at low precision instead (absmax int8 or int4 codes per (token, head), K and V
// separately).
//
// Pages are written with non-temporal stores: the pool (hundreds of MB) is not read again
// until the next decode attention, and ordinary stores leave it as dirty lines in the
// MALL whose write-back then competes with that attention's reads (measured on the
// Qwen-3-8B-like layer: attention right after compaction 142 -> 113 us, compaction
// 240 -> 255 us).
//
// Work units are destination pages of 16 slots.  Copy units (a pair's pool pages, then
// its ring pages) go to compact_copy_kernel and low-precision pages to
// compact_quant_kernel; in both, each wave owns one contiguous run of units, so it
// finds its first pair once and then walks pairs in order, and a page is handled by
// one wave (K rows straight through, V transposed through the wave's own LDS tile),
// with no work-group barrier.
#include "kvp_internal.h"

namespace kvp {

constexpr int CMP_THREADS = 256;
constexpr int CMP_GRID = 2048;
constexpr int CPY_WAVES = CMP_THREADS / 64;
constexpr int PLAN_THREADS = 1024;

struct CompactArgs {
  const void* k;
  const void* v;
  int T, d, num_pairs;
  const int* kept_idx;
  const int* kept_count;
  const float* scores;
  int64_t ld_s;
  int demote;
  kvp_paged_kv kv;
  kvp_ring ring;
  int has_ring;
  int* ws;  // npool | pbase | nring | n8 | p8base | wbase (np+1) | tmp
};

__device__ __forceinline__ int* ws_npool(const CompactArgs& a) { return a.ws; }
__device__ __forceinline__ int* ws_pbase(const CompactArgs& a) { return a.ws + a.num_pairs; }
__device__ __forceinline__ int* ws_nring(const CompactArgs& a) { return a.ws + 2 * a.num_pairs; }
__device__ __forceinline__ int* ws_n8(const CompactArgs& a) { return a.ws + 3 * a.num_pairs; }
__device__ __forceinline__ int* ws_p8base(const CompactArgs& a) { return a.ws + 4 * a.num_pairs; }
__device__ __forceinline__ int* ws_wbase(const CompactArgs& a) { return a.ws + 5 * a.num_pairs; }
__device__ __forceinline__ int* ws_tmp(const CompactArgs& a) { return a.ws + 6 * a.num_pairs + 1; }

// first index i in [lo, hi) with arr[i] >= x (arr ascending), hi if none
__device__ __forceinline__ int lower_bound_i(const int* arr, int lo, int hi, int x) {
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (arr[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(PLAN_THREADS) void compact_plan_kernel(CompactArgs a) {
  const int np = a.num_pairs;
  int* npool = ws_npool(a);
  int* pbase = ws_pbase(a);
  int* nring = ws_nring(a);
  int* n8 = ws_n8(a);
  int* p8base = ws_p8base(a);
  int* wbase = ws_wbase(a);
  __shared__ int tmp[PLAN_THREADS / 64];
  const int w = a.has_ring ? a.ring.window : 0;
  int errbits = 0;
  for (int p = threadIdx.x; p < np; p += blockDim.x) {
    const int cnt = a.kept_count[p];
    const int* idx = a.kept_idx + (int64_t)p * a.T;
    int nr = 0;
    if (a.has_ring) nr = cnt - lower_bound_i(idx, 0, cnt, a.T - w);
    int npl = cnt - nr;
    int pages = cdiv(npl, PAGE);
    if (pages > a.kv.max_pages_per_pair) {
      errbits |= KVP_ERR_TABLE_FULL;
      pages = a.kv.max_pages_per_pair;
      npl = pages * PAGE;
    }
    int ne = a.demote ? (a.T - cnt) : 0;
    int pages8 = cdiv(ne, PAGE);
    if (a.demote && pages8 > a.kv.max_pages8_per_pair) {
      errbits |= KVP_ERR_POOL8_FULL;
      pages8 = a.kv.max_pages8_per_pair;
      ne = pages8 * PAGE;
    }
    npool[p] = npl;
    nring[p] = nr;
    n8[p] = ne;
    pbase[p] = pages;
    p8base[p] = pages8;
  }
  __syncthreads();
  const int total = block_excl_scan_lds(pbase, np, tmp);
  const int total8 = block_excl_scan_lds(p8base, np, tmp);
  const int rpages = w / PAGE;
  for (int p = threadIdx.x; p <= np; p += blockDim.x) {
    if (p == np) {
      wbase[np] = 0;
      continue;
    }
    int pages = cdiv(npool[p], PAGE);
    if (pbase[p] + pages > a.kv.num_pages) {
      errbits |= KVP_ERR_POOL_FULL;
      pages = max(0, a.kv.num_pages - pbase[p]);
      npool[p] = min(npool[p], pages * PAGE);
    }
    int pages8 = cdiv(n8[p], PAGE);
    if (a.demote && p8base[p] + pages8 > a.kv.num_pages8) {
      errbits |= KVP_ERR_POOL8_FULL;
      pages8 = max(0, a.kv.num_pages8 - p8base[p]);
      n8[p] = min(n8[p], pages8 * PAGE);
    }
    a.kv.length[p] = npool[p];
    if (a.kv.num_pages8 > 0) a.kv.length8[p] = a.demote ? n8[p] : 0;
    wbase[p] = pages + rpages;  // copy units; int8 pages are numbered by p8base
  }
  __syncthreads();
  block_excl_scan_lds(wbase, np + 1, tmp);
  if (threadIdx.x == 0) {
    a.kv.page_top[0] = min(total, a.kv.num_pages);
    if (a.kv.num_pages8 > 0) a.kv.page8_top[0] = a.demote ? min(total8, a.kv.num_pages8) : 0;
  }
  if (errbits) atomicOr(a.kv.err, errbits);
}

template <typename E>
__device__ __forceinline__ float elem_to_f32(E x);
template <>
__device__ __forceinline__ float elem_to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }
template <>
__device__ __forceinline__ float elem_to_f32<float>(float x) { return x; }

// Slot of ring page r, lane i: the ring holds positions [T - w, T), position t in slot
// t mod w.  Returns the source row (t if t was kept, else -1) for lanes < PAGE.
__device__ __forceinline__ int ring_src(const CompactArgs& a, const int* idx, int cnt, int nr, int r,
                                        int i, int w) {
  const int slot = r * PAGE + i;
  const int base = a.T - w;
  const int t = base + (((slot - base) % w) + w) % w;
  int s = -1;
  if (t >= 0) {
    const int lo = cnt - nr;
    const int at = lower_bound_i(idx, lo, cnt, t);
    if (at < cnt && idx[at] == t) s = t;
  }
  return s;
}

template <typename E, int D>
__global__ __launch_bounds__(CMP_THREADS) void compact_copy_kernel(CompactArgs a) {
  constexpr int EPC = 16 / sizeof(E);    // elements per 16-byte chunk
  constexpr int CPR = D / EPC;           // chunks per K row
  constexpr int NCH = PAGE * CPR;        // chunks per page (128 .. 512)
  constexpr int NPL = NCH / 64;          // chunks per lane
  constexpr int TCH = PAGE / EPC;        // chunks per V^T row (one dim, 16 slots)
  __shared__ __attribute__((aligned(16))) E tile[CPY_WAVES][PAGE * D];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  E* vt = tile[wid];
  const int np = a.num_pairs;
  const int* wbase = ws_wbase(a);
  const int total = wbase[np];
  const int nw = gridDim.x * CPY_WAVES;
  const int per = cdiv(total, nw);
  int u = (blockIdx.x * CPY_WAVES + wid) * per;
  const int uend = min(total, u + per);
  if (u >= uend) return;
  const int w = a.has_ring ? a.ring.window : 0;
  const int rpages = w / PAGE;
  int p = upper_segment(wbase, np, u);
  int pb = wbase[p], pe = wbase[p + 1];
  for (; u < uend; ++u) {
    while (u >= pe) {  // next pair (units of a pair are contiguous)
      ++p;
      pb = pe;
      pe = wbase[p + 1];
    }
    const int local = u - pb;
    const int npl = ws_npool(a)[p];
    const int pages = cdiv(npl, PAGE);
    const int cnt = a.kept_count[p];
    const int* idx = a.kept_idx + (int64_t)p * a.T;
    const E* ksrc = reinterpret_cast<const E*>(a.k) + (int64_t)p * a.T * D;
    const E* vsrc = reinterpret_cast<const E*>(a.v) + (int64_t)p * a.T * D;
    E* kdst;
    E* vdst;
    int s = -1;  // lanes < PAGE: source row of slot `lane`
    if (local < pages) {
      const int dst = ws_pbase(a)[p] + local;
      if (lane < PAGE) {
        if (local * PAGE + lane < npl) s = idx[local * PAGE + lane];
        a.kv.page_pos[(int64_t)dst * PAGE + lane] = s;
      }
      if (lane == 0) a.kv.block_table[(int64_t)p * a.kv.max_pages_per_pair + local] = dst;
      kdst = reinterpret_cast<E*>(a.kv.k_pages) + (int64_t)dst * PAGE * D;
      vdst = reinterpret_cast<E*>(a.kv.v_pages) + (int64_t)dst * PAGE * D;
    } else {
      const int r = local - pages;
      if (lane < PAGE) {
        s = ring_src(a, idx, cnt, ws_nring(a)[p], r, lane, w);
        const int slot = r * PAGE + lane;
        a.ring.pos[(int64_t)p * w + slot] = s;
        a.ring.score[(int64_t)p * w + slot] = (s >= 0) ? a.scores[(int64_t)p * a.ld_s + s] : 0.f;
      }
      const int64_t off = ((int64_t)p * rpages + r) * PAGE * D;
      kdst = reinterpret_cast<E*>(a.ring.k) + off;
      vdst = reinterpret_cast<E*>(a.ring.v) + off;
    }
    // gather: chunk c = lane + 64 i is row c / CPR, columns (c % CPR) * EPC ..
    u32x4 kx[NPL], vx[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int c = lane + 64 * i, row = c / CPR, col = (c % CPR) * EPC;
      const int sr = __shfl(s, row);
      kx[i] = u32x4{0u, 0u, 0u, 0u};
      vx[i] = u32x4{0u, 0u, 0u, 0u};
      if (sr >= 0) {
        kx[i] = *reinterpret_cast<const u32x4*>(ksrc + (int64_t)sr * D + col);
        vx[i] = *reinterpret_cast<const u32x4*>(vsrc + (int64_t)sr * D + col);
      }
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int c = lane + 64 * i;
      __builtin_nontemporal_store(kx[i], reinterpret_cast<u32x4*>(kdst + c * EPC));
      *reinterpret_cast<u32x4*>(vt + c * EPC) = vx[i];  // V rows [16][D] in LDS
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // V^T: chunk c = lane + 64 i is dim c / TCH, slots (c % TCH) * EPC ..
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int c = lane + 64 * i, dd = c / TCH, t0 = (c % TCH) * EPC;
      E tmp[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) tmp[e] = vt[(t0 + e) * D + dd];
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(tmp), reinterpret_cast<u32x4*>(vdst + dd * PAGE + t0));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
}

// int8 pages: unit u is int8 page u of the pool; its pair is the last one whose page
// base is <= u (pairs without int8 pages share the next pair's base).
// Low-precision pages, one wave per page over a contiguous range of pages (like the
// copy kernel): the 16 source rows of K and of V are gathered as 16-byte chunks (a
// row's chunks sit in consecutive lanes), each row's absmax is a shuffle reduction over
// those lanes, K codes go straight to the token-major page, V codes through this wave's
// LDS tile to the dim-major page.
// Codes of N values of one row for the row scale s, bit for bit clamp(rint(fl(x / s)),
// -qmax, qmax) with fl the correctly rounded fp32 quotient, at a fraction of N divisions'
// cost.  inv is an approximate 1 / s (0 when s = 0, whose row is all zeros).  y = x * inv
// is within 127 (2^-22 + 2^-24) < 2^-14.7 of x / s and fl(x / s) within 2^-18 of x / s,
// so unless y lies within 2^-12 of a half-integer both round to the same integer; those
// values (rare: a branch per value, taken when any lane needs it) are divided exactly.  The code is the
// low byte of the bits of y + 1.5 2^23 (that addition rounds to the nearest integer,
// ties to even, and keeps it in the low mantissa bits).  No clamp is needed: with
// s = fl(max |x| / qmax), |x / s| <= qmax (1 + 2^-23) and |y| < qmax + 1/2.
template <int N>
__device__ __forceinline__ void quant_codes_fast(const float (&x)[N], float s, float inv,
                                                 uint32_t (&bits)[N]) {
  constexpr float M = 12582912.0f;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float y = x[e] * inv;
    float t = y + M;
    if (fabsf(y - (t - M)) > 0.5f - 0x1p-12f) t = rintf(x[e] / s) + M;
    bits[e] = __float_as_uint(t);
  }
}

// max over each aligned group of G lanes (G = 8, 16 or 32), every lane of the group
// receiving it: DPP quad swaps and row mirrors, and one cross-row exchange for G = 32.
template <int G>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)));
  if constexpr (G >= 16)
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false)));
  if constexpr (G >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  return v;
}

// F8: E4M3 codes (BITS = 8): scale = absmax / 448, each code the E4M3 rounding of the
// correctly rounded quotient (an IEEE division per element; this format is not tuned).
template <typename E, int D, int BITS, bool F8 = false>
__global__ __launch_bounds__(CMP_THREADS) void compact_quant_kernel(CompactArgs a) {
  static_assert(!F8 || BITS == 8, "fp8 codes are one byte");
  constexpr int EPC = 16 / sizeof(E);  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;         // chunks per row (8 .. 32; divides 64)
  constexpr int NPL = PAGE * CPR / 64; // chunks per lane
  constexpr float QMAX = F8 ? 448.0f : (BITS == 4 ? 7.0f : 127.0f);
  constexpr int CB = EPC * BITS / 8;   // code bytes per chunk (2 .. 8)
  __shared__ int8_t vcodes[CPY_WAVES][PAGE * D];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int8_t* vc = vcodes[wid];
  const int np = a.num_pairs;
  const int* p8base = ws_p8base(a);
  const int total = a.kv.page8_top[0];
  const int nw = gridDim.x * CPY_WAVES;
  const int per = cdiv(total, nw);
  int u = (blockIdx.x * CPY_WAVES + wid) * per;
  const int uend = min(total, u + per);
  if (u >= uend) return;
  int p = upper_segment(p8base, np, u);
  int pb = p8base[p];
  int pe = (p + 1 < np) ? p8base[p + 1] : total;
  for (; u < uend; ++u) {
    while (u >= pe) {  // next pair (a pair's pages are contiguous)
      ++p;
      pb = pe;
      pe = (p + 1 < np) ? p8base[p + 1] : total;
    }
    const int j8 = u - pb;
    const int ne = ws_n8(a)[p];
    if (j8 >= cdiv(ne, PAGE)) continue;  // uniform across the wave
    const int cnt = a.kept_count[p];
    const int* idx = a.kept_idx + (int64_t)p * a.T;
    const E* ksrc = reinterpret_cast<const E*>(a.k) + (int64_t)p * a.T * D;
    const E* vsrc = reinterpret_cast<const E*>(a.v) + (int64_t)p * a.T * D;
    int s = -1;  // lanes < PAGE: source row of slot `lane`
    if (lane < PAGE) {
      if (j8 * PAGE + lane < ne) s = idx[cnt + j8 * PAGE + lane];
      a.kv.page8_pos[(int64_t)u * PAGE + lane] = s;
    }
    if (lane == 0) a.kv.block_table8[(int64_t)p * a.kv.max_pages8_per_pair + j8] = u;
    u32x4 kx[NPL], vx[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int c = lane + 64 * i, row = c / CPR, col = (c % CPR) * EPC;
      const int sr = __shfl(s, row);
      kx[i] = u32x4{0u, 0u, 0u, 0u};
      vx[i] = u32x4{0u, 0u, 0u, 0u};
      if (sr >= 0) {
        kx[i] = *reinterpret_cast<const u32x4*>(ksrc + (int64_t)sr * D + col);
        vx[i] = *reinterpret_cast<const u32x4*>(vsrc + (int64_t)sr * D + col);
      }
    }
    int8_t* kdst = a.kv.k8_pages + (int64_t)u * PAGE * D * BITS / 8;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int c = lane + 64 * i, row = c / CPR, col = (c % CPR) * EPC;
      const E* ke = reinterpret_cast<const E*>(&kx[i]);
      const E* ve = reinterpret_cast<const E*>(&vx[i]);
      float kf[EPC], vf[EPC], ka = 0.f, va = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        kf[e] = elem_to_f32<E>(ke[e]);
        vf[e] = elem_to_f32<E>(ve[e]);
        ka = fmaxf(ka, fabsf(kf[e]));
        va = fmaxf(va, fabsf(vf[e]));
      }
      // the row's CPR chunks are CPR aligned lanes
      ka = group_max<CPR>(ka);
      va = group_max<CPR>(va);
      const float kscale = ka / QMAX, vscale = va / QMAX;
      const float kinv = kscale > 0.f ? __builtin_amdgcn_rcpf(kscale) : 0.f;
      const float vinv = vscale > 0.f ? __builtin_amdgcn_rcpf(vscale) : 0.f;
      uint32_t kb[EPC], vb[EPC];
      if constexpr (F8) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          kb[e] = fp8_quant_code(kf[e], kscale);
          vb[e] = fp8_quant_code(vf[e], vscale);
        }
      } else {
        quant_codes_fast<EPC>(kf, kscale, kinv, kb);
        quant_codes_fast<EPC>(vf, vscale, vinv, vb);
      }
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if constexpr (BITS == 8) w[e / 4] |= (kb[e] & 0xffu) << (8 * (e % 4));
        else w[e / 8] |= (kb[e] & 0xfu) << (4 * (e % 8));
        vc[row * D + col + e] = static_cast<int8_t>(vb[e]);
      }
      int8_t* kd = kdst + (row * D + col) * BITS / 8;
      if constexpr (CB == 8) __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(kd));
      else if constexpr (CB == 4) __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(kd));
      else __builtin_nontemporal_store(static_cast<uint16_t>(w[0]), reinterpret_cast<uint16_t*>(kd));
      if ((c % CPR) == 0) {
        a.kv.k8_scale[(int64_t)u * PAGE + row] = kscale;
        a.kv.v8_scale[(int64_t)u * PAGE + row] = vscale;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // V^T page: dim dd's 16 codes (int8: 16 bytes; int4: 8 bytes, token 2i in the low nibble)
    int8_t* vdst = a.kv.v8_pages + (int64_t)u * PAGE * D * BITS / 8;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int dd = lane + 64 * k;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = 0; t < PAGE; ++t) {
        const uint32_t code = static_cast<uint32_t>(static_cast<int>(vc[t * D + dd]));
        if constexpr (BITS == 8) w[t / 4] |= (code & 0xffu) << (8 * (t % 4));
        else w[t / 8] |= (code & 0xfu) << (4 * (t % 8));
      }
      if constexpr (BITS == 8) __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(vdst + dd * PAGE));
      else __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(vdst + dd * (PAGE / 2)));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
}

}  // namespace kvp

using namespace kvp;

extern "C" size_t kvp_compact_workspace_size(int32_t B, int32_t Hkv) {
  if (B <= 0 || Hkv <= 0) return 0;
  const size_t np = (size_t)B * Hkv;
  return ((6 * np + 1 + 64) * sizeof(int) + 255) & ~(size_t)255;
}

kvp_status kvp_launch_compact(const void* k, const void* v, int num_pairs, int T, int d,
                              const int* kept_idx, const int* kept_count, const float* scores,
                              int64_t ld_s, int demote, const kvp_paged_kv* kv,
                              const kvp_ring* ring, void* ws, hipStream_t stream) {
  CompactArgs a;
  a.k = k;
  a.v = v;
  a.T = T;
  a.d = d;
  a.num_pairs = num_pairs;
  a.kept_idx = kept_idx;
  a.kept_count = kept_count;
  a.scores = scores;
  a.ld_s = ld_s;
  a.demote = demote;
  a.kv = *kv;
  a.has_ring = ring != nullptr;
  if (ring) a.ring = *ring;
  else a.ring = kvp_ring{};
  a.ws = reinterpret_cast<int*>(ws);
  hipLaunchKernelGGL(compact_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, a);
  KVP_LAUNCH_CHECK();
  const bool bf = kv->dtype == KVP_BF16;
  if (bf && d == 128)
    hipLaunchKernelGGL((compact_copy_kernel<uint16_t, 128>), dim3(CMP_GRID), dim3(CMP_THREADS), 0, stream, a);
  else if (bf)
    hipLaunchKernelGGL((compact_copy_kernel<uint16_t, 64>), dim3(CMP_GRID), dim3(CMP_THREADS), 0, stream, a);
  else if (d == 128)
    hipLaunchKernelGGL((compact_copy_kernel<float, 128>), dim3(CMP_GRID), dim3(CMP_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((compact_copy_kernel<float, 64>), dim3(CMP_GRID), dim3(CMP_THREADS), 0, stream, a);
  KVP_LAUNCH_CHECK();
  if (demote) {
    const bool i4 = lp_bits_of(*kv) == 4, f8 = lp_is_fp8(*kv);
    const dim3 g(CMP_GRID), b(CMP_THREADS);
#define KVP_QUANT(E, DD)                                                                           \
  do {                                                                                             \
    if (i4) hipLaunchKernelGGL((compact_quant_kernel<E, DD, 4>), g, b, 0, stream, a);              \
    else if (f8) hipLaunchKernelGGL((compact_quant_kernel<E, DD, 8, true>), g, b, 0, stream, a);   \
    else hipLaunchKernelGGL((compact_quant_kernel<E, DD, 8>), g, b, 0, stream, a);                 \
  } while (0)
    if (bf) {
      if (d == 128) KVP_QUANT(uint16_t, 128);
      else KVP_QUANT(uint16_t, 64);
    } else {
      if (d == 128) KVP_QUANT(float, 128);
      else KVP_QUANT(float, 64);
    }
#undef KVP_QUANT
    KVP_LAUNCH_CHECK();
  }
  return KVP_OK;
}
