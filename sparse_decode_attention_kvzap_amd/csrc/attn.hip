// GQA decode attention over the kept entries of the paged cache (gfx950).
//
// Method: KVzap digest (max5.ai), key points -- pruning shortens the sequence axis,
// which GQA alone does not; the attention reads only the kept entries.  BeaconKV
// briefing (jiinsi.com), body -- beacon entries at full precision and the others at
// low precision are read in one attention.
//
// Work decomposition (split-K, evenly balanced), two kernels:
//   Every pair (b, h_kv) contributes a "region A" of virtual pages (its pool pages,
//   then its ring pages, padded to an even count) and, when a low-precision pool exists,
//   a "region B" (its int8, int4 or fp8 pages, padded to even).  The A regions are
//   concatenated into one page sequence and the B regions into another; each sequence
//   is cut into one contiguous unit per wave.  A wave walks its units 32 tokens (two
//   pages) at a time and writes one partial (max, sum, output) record per segment (the
//   part of a region inside a unit); a pair whose whole sequence lies in one segment is
//   finished by that wave.  The merge kernel (one wave per pair and query head) combines
//   a pair's records in page order with a log-sum-exp merge, so the result is
//   deterministic; the kernel boundary makes the records visible (no atomics, no cache
//   maintenance).  Record slot of segment (region s, unit u) = s + u: consecutive
//   segments of a sequence advance s or u (or both), so slots are unique and a region's
//   records are consecutive.
//
// Fused decode step (kvp_decode_step; DeInfer methodology (b): a fixed-address step
// replayed from a graph): the stream kernel reads the cache as the delayed step will
// leave it -- the token leaving the ring slot counts iff it is retained, the new token is
// one more one-row virtual page -- without writing it; with an MLP scorer, waves 1..3 of
// every work-group compute the split-K slices of the new tokens' first layer while wave 0
// builds the plan; the merge kernel then finishes the scores and applies the step on
// waves of its own, after every read of the ring is done.
//
// Per 32-token step (bf16, head dim D, g query heads of one KV head):
//   S^T[32 tok x 16 heads] = K . Q^T on 16x16x32 bf16 MFMA (exact products, fp32
//   accumulation).  The K rows given to the two 16-row MFMA tiles are interleaved
//   so that each lane ends up holding the scores of 8 consecutive tokens of one head,
//   which is exactly the B-operand layout of the P.V MFMA that follows.
//   O^T[D x 16 heads] += V^T . P^T on MFMA, with P split into bf16 hi + lo parts so
//   the probabilities keep ~16 significant bits (V is exact in bf16).
//   V pages are stored dim-major ([d][16]) so V^T fragments are plain 16-byte loads.
// The bf16 stream keeps one step of K/V loads in flight, issued unconditionally so the
// compiler's wait counts stay exact (QK waits for K while V is still in flight), and
// looks two segments ahead: the next segments' block-table entries are requested while
// the current one streams and the next pair's queries with its first K, so crossing from
// one pair to the next costs no memory round trip.
#include "small_gemm.h"
#include "step_core.h"

namespace kvp {

constexpr int ATTN_WG_WAVES = 4;
constexpr int ATTN_GRID = 256;  // one work-group (4 waves) per CU on a 256-CU part
// int4 and fp8 pools run two work-groups per CU (two waves per SIMD): a 32-token step of
// their codes costs more instructions than the bytes it moves (nibble decode and offset
// terms; the E4M3 -> bf16 rebuild), and one wave per SIMD leaves its MFMA/VALU latencies
// exposed (measured on the BeaconKV cache: int4 194 -> 171 us, fp8 297 -> 255 us).  Every
// other cache keeps one wave per SIMD (the bf16 and int8 streams ran 1-4% slower with two).
constexpr int ATTN_MAX_WPE = 2;
constexpr int ATTN_MAX_NWAVES = ATTN_MAX_WPE * ATTN_GRID * ATTN_WG_WAVES;
// Register sets of code-pool loads in flight per wave (two 32-token steps): more sets
// (4 or 6) made the int4 stream 5-15% slower, fewer leave the loads exposed.
constexpr int ATTN_LP_SETS = 2;
static_assert(ATTN_GRID % 8 == 0, "units are numbered per XCD (8 XCDs)");

struct AttnArgs {
  const void* q;
  float* out;
  int B, Hkv, Hq, g, D;
  kvp_paged_kv kv;
  kvp_ring ring;
  int has_ring;
  float scale_log2;  // sm_scale * log2(e)
  int* plan;         // page prefix P[0..nseg], written by work-group 0 for the merge kernel
  int nw;            // waves of the streaming kernel
  float* part;       // records, rec_floats each
  int rec_floats;    // g * (D + 2) rounded up to 4: o[g][D], then m[g], then l[g]
  // Fused decode step (fstep = 1, bf16 pool with a ring, no low-precision pool): the
  // attention reads the cache as the delayed step st would leave it -- the token leaving
  // ring slot p mod window counts iff it is retained, the new token (st.k_new, st.v_new)
  // is one more virtual page of its pair -- and the merge kernel then applies the step.
  int fstep;
  StepArgs st;
  // Fused decode step with the MLP scorer (fgemm = 1): the split-K slices of the new
  // tokens' first layer, taken by waves 1..3 of every work-group while wave 0 builds the
  // plan; the merge kernel's step waves add them up (st.part = gm.part).
  int fgemm;
  SmallGemm gm;
  // Plan in global memory (gplan = 1, when P and Lens would not fit in LDS): written by
  // decode_attn_plan_kernel before the stream kernel -- P[0..nseg] at plan, Lens at
  // plan + nseg + 2 -- and read from there by every wave.
  int gplan;
};

// -------------------------------------------------------------------------------
// Plan: page prefix P[] over the regions, computed by every work-group into LDS (one load
// per region, a wave or work-group scan).
// -------------------------------------------------------------------------------
__device__ __forceinline__ int plan_regions(const AttnArgs& a) {
  return (a.kv.num_pages8 > 0 ? 2 : 1) * a.kv.num_pairs;
}

__device__ __forceinline__ int region_pages_of(int len, int extra) { return (cdiv(len, PAGE) + extra + 1) & ~1; }

// Wave 0: P[0] = 0, P[s + 1] = P[s] + pages of region s.  Each lane takes a run of
// regions; lengths are requested eight at a time so the loads overlap.
// The A regions' pool lengths go to Lens[] on the way; with a fused step, bit 31 of
// Lens[s] says whether the token leaving pair s's ring slot `slot` is retained (its
// position >= 0 and score >= tau), and each A region has one more page (the new token).
constexpr int LEN_MASK = 0x7fffffff;
// Regions [s0, s1) of one thread: page counts to P[s + 1] (and pool lengths to Lens);
// returns their sum.  Loads are requested eight regions at a time.
__device__ __forceinline__ int plan_counts(const AttnArgs& a, int* P, int* Lens, int s0, int s1, int slot,
                                           float tau) {
  const int np = a.kv.num_pairs;
  const int nring = a.has_ring ? a.ring.window / PAGE + a.fstep : 0;
  int sum = 0;
  for (int b = s0; b < s1; b += 8) {
    int v[8];
    int rpos[8];
    float rsc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = b + i;
      v[i] = 0;
      rpos[i] = -1;
      rsc[i] = 0.f;
      if (s < s1) v[i] = (s < np) ? a.kv.length[s] : a.kv.length8[s - np];
      if (a.fstep && s < s1) {
        rpos[i] = a.ring.pos[(int64_t)s * a.ring.window + slot];
        rsc[i] = a.ring.score[(int64_t)s * a.ring.window + slot];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = b + i;
      if (s < s1) {
        if (s < np) Lens[s] = v[i] | ((rpos[i] >= 0 && rsc[i] >= tau) ? (int)0x80000000u : 0);
        const int n = region_pages_of(v[i], s < np ? nring : 0);
        P[s + 1] = n;
        sum += n;
      }
    }
  }
  return sum;
}

// Regions [s0, s1) of one thread: P[s + 1] = run + the counts up to s.
__device__ __forceinline__ void plan_prefix(int* P, int s0, int s1, int run) {
  for (int b = s0; b < s1; b += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (b + i < s1) ? P[b + i + 1] : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (b + i < s1) {
        run += v[i];
        P[b + i + 1] = run;
      }
    }
  }
}

__device__ __forceinline__ void compute_plan(const AttnArgs& a, int* P, int* Lens, int nseg, int slot,
                                             float tau) {
  const int lane = threadIdx.x & 63;
  const int per = cdiv(nseg, 64);
  const int s0 = min(nseg, lane * per), s1 = min(nseg, s0 + per);
  const int sum = plan_counts(a, P, Lens, s0, s1, slot, tau);
  plan_prefix(P, s0, s1, wave_incl_scan(sum) - sum);
  if (lane == 0) P[0] = 0;
}

// The same plan by all NT threads of the work-group (every thread must call it): each
// takes nseg / NT regions, so many pairs cost NT / 64 times fewer round trips.  wsum:
// NT / 64 ints of LDS.
template <int NT>
__device__ __forceinline__ void compute_plan_wg(const AttnArgs& a, int* P, int* Lens, int nseg, int slot,
                                                float tau, int* wsum) {
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int per = cdiv(nseg, NT);
  const int s0 = min(nseg, t * per), s1 = min(nseg, s0 + per);
  const int sum = plan_counts(a, P, Lens, s0, s1, slot, tau);
  const int incl = wave_incl_scan(sum);
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wid; ++w) base += wsum[w];
  plan_prefix(P, s0, s1, base + incl - sum);
  if (t == 0) P[0] = 0;
}

// Largest s in [lo, hi) with P[s] <= x (P nondecreasing, P[lo] <= x): one LDS read and
// one ballot per level of 64.
__device__ __forceinline__ int seg_search(const int* P, int lo, int hi, int x) {
  const int lane = threadIdx.x & 63;
  int n = hi - lo;
  while (n > 64) {
    const int stride = cdiv(n, 64);
    const int s = lo + lane * stride;
    const uint64_t m = __ballot(s < hi && P[s] <= x);
    const int k = 63 - __builtin_clzll(m);
    lo += k * stride;
    hi = min(hi, lo + stride);
    n = hi - lo;
  }
  const int s = lo + lane;
  const uint64_t m = __ballot(s < hi && P[s] <= x);
  return lo + (63 - __builtin_clzll(m));
}

// Units and records.  Sequence A is regions [0, np) of P, sequence B regions [np, 2 np);
// each is cut into nw units of s pages (the last ones short or empty).
struct Plan {
  const int* P;
  int np, nw;
  int sA, sB;  // unit sizes
  int NA;      // pages of sequence A (= P[np])
  int baseB;   // first record slot of sequence B
  int lp;
};

__device__ __forceinline__ int unit_size(int N, int nw) { return N > 0 ? ((cdiv(N, nw) + 1) & ~1) : 0; }

__device__ __forceinline__ Plan make_plan(const int* P, int np, int nw, bool lp) {
  Plan pl;
  pl.P = P;
  pl.np = np;
  pl.nw = nw;
  pl.lp = lp ? 1 : 0;
  pl.NA = P[np];
  pl.sA = unit_size(pl.NA, nw);
  pl.sB = lp ? unit_size(P[2 * np] - pl.NA, nw) : 0;
  pl.baseB = np + nw;
  return pl;
}

// Records of region s (first unit in uf): the units it intersects.
__device__ __forceinline__ int region_records(const Plan& pl, int s, int& uf) {
  const bool b = s >= pl.np;
  const int base = b ? pl.NA : 0, us = b ? pl.sB : pl.sA;
  const int p0 = pl.P[s] - base, p1 = pl.P[s + 1] - base;
  if (p1 <= p0) {
    uf = 0;
    return 0;
  }
  uf = p0 / us;
  return (p1 - 1) / us - uf + 1;
}

__device__ __forceinline__ int pair_records(const Plan& pl, int pair) {
  int uf;
  int n = region_records(pl, pair, uf);
  if (pl.lp) n += region_records(pl, pl.np + pair, uf);
  return n;
}

struct SegDesc {
  int s;         // region index in P
  int vlo, vhi;  // pages of the region covered by the segment
  int u;         // unit
  int rev;       // walk backwards
  int ok;        // 1: a segment; 0: no more work; -1: not looked up yet
};

__device__ __forceinline__ int slot_of(const Plan& pl, const SegDesc& d) {
  return d.s < pl.np ? d.s + d.u : pl.baseB + (d.s - pl.np) + d.u;
}

// The segments of one wave's unit of a sequence, in walk order.  Odd units walk
// backwards: with all 1024 streams walking forward at a fixed distance, one keep ratio
// of the Qwen-3-8B-like cache ran 10% slower (HBM channel conflicts of the regular
// stride); opposite directions remove that.  The order only changes rounding inside a
// record.
struct UnitIter {
  int X0, X1, rev;  // the unit's pages in P coordinates
  int r, r_end;     // next region to emit, last region (walk order)
  int have;
};

__device__ __forceinline__ void iter_init(UnitIter& it, const Plan& pl, bool seqB, int u) {
  const int base = seqB ? pl.NA : 0, us = seqB ? pl.sB : pl.sA;
  const int N = seqB ? pl.P[2 * pl.np] - pl.NA : pl.NA;
  const int r0 = seqB ? pl.np : 0;
  it.have = 0;
  const int x0 = u * us, x1 = min(N, x0 + us);
  if (us == 0 || x1 <= x0) return;
  it.X0 = base + x0;
  it.X1 = base + x1;
  it.rev = u & 1;
  const int rf = seg_search(pl.P, r0, r0 + pl.np, it.X0);
  const int rl = seg_search(pl.P, r0, r0 + pl.np, it.X1 - 1);
  it.r = it.rev ? rl : rf;
  it.r_end = it.rev ? rf : rl;
  it.have = 1;
}

__device__ __forceinline__ SegDesc iter_next_seg(UnitIter& it, const Plan& pl, int u) {
  SegDesc d;
  d.ok = 0;
  while (it.have) {
    const int r = it.r;
    if (r == it.r_end) it.have = 0;
    else it.r += it.rev ? -1 : 1;
    const int p0 = __builtin_amdgcn_readfirstlane(pl.P[r]), p1 = __builtin_amdgcn_readfirstlane(pl.P[r + 1]);
    if (p1 > p0) {
      d.s = r;
      d.vlo = max(it.X0, p0) - p0;
      d.vhi = min(it.X1, p1) - p0;
      d.u = u;
      d.rev = it.rev;
      d.ok = 1;
      return d;
    }
  }
  return d;
}

// -------------------------------------------------------------------------------
// bf16 region-A step machinery
// -------------------------------------------------------------------------------
template <int D>
struct Bf16Frags {
  u32x4 kA[D / 32];  // K rows for score tile A (this lane's row, D/4 elements)
  u32x4 kB[D / 32];  // K rows for score tile B
  u32x4 v[D / 16];   // V^T fragments, one per 16-wide output tile
  u32x4 rp0, rp1;    // ring pages: the positions of this lane's 8 tokens (-1 = empty)
};

struct PageRef {
  const uint16_t* k;  // K page base
  const uint16_t* v;  // V^T page base
  int kind;           // 0 main, 1 ring, 2 padding, 3 the new token of a fused step
  int nvalid;         // main: valid slots; ring: ring page index
  int rowmask;        // K row r of the page is row (r & rowmask): 15, or 0 for kind 3
  uint32_t drop;      // ring: slots hidden although occupied (the leaving token, not retained)
};

// Fused step: the ring slot being turned over (page fs.rp, slot fs.rs; fs.rp = -1 when
// there is no fused step) and whether the leaving token of the current pair is retained.
struct FStep {
  int rp, rs;
};

// Page v of region A of `pair` (walk position w, for the block-table chunk in bt).
template <int D>
__device__ __forceinline__ PageRef region_a_page(const AttnArgs& a, int pair, int v, int w, int bt, int npm,
                                                 int len, int nring, FStep fs, bool app) {
  PageRef r;
  r.rowmask = 15;
  r.drop = 0u;
  if (v < npm) {
    const int pg = __builtin_amdgcn_readlane(bt, w & 63);
    r.k = reinterpret_cast<const uint16_t*>(a.kv.k_pages) + (int64_t)pg * PAGE * D;
    r.v = reinterpret_cast<const uint16_t*>(a.kv.v_pages) + (int64_t)pg * PAGE * D;
    r.kind = 0;
    r.nvalid = min(PAGE, len - v * PAGE);
  } else if (v < npm + nring) {
    const int rp = v - npm;
    const int64_t off = ((int64_t)pair * nring + rp) * PAGE * D;
    r.k = reinterpret_cast<const uint16_t*>(a.ring.k) + off;
    r.v = reinterpret_cast<const uint16_t*>(a.ring.v) + off;
    r.kind = 1;
    r.nvalid = rp;
    if (rp == fs.rp && !app) r.drop = 1u << fs.rs;
  } else if (fs.rp >= 0 && v == npm + nring) {
    // the new token: K row and V values of the pair in k_new / v_new (every K row of
    // the page reads row 0; only token 0 is valid)
    r.k = reinterpret_cast<const uint16_t*>(a.st.k_new) + (int64_t)pair * D;
    r.v = reinterpret_cast<const uint16_t*>(a.st.v_new) + (int64_t)pair * D;
    r.kind = 3;
    r.nvalid = 1;
    r.rowmask = 0;
  } else {
    // padding: its (ignored) loads read page X, which is always a full page -- except
    // with a fused step, where X may be the one-row new-token page; then they read the
    // pair's first ring page instead
    r.k = nullptr;
    r.v = nullptr;
    if (fs.rp >= 0) {
      const int64_t off = (int64_t)pair * nring * PAGE * D;
      r.k = reinterpret_cast<const uint16_t*>(a.ring.k) + off;
      r.v = reinterpret_cast<const uint16_t*>(a.ring.v) + off;
    }
    r.kind = 2;
    r.nvalid = 0;
  }
  return r;
}

// The two pages of step k of a segment (X the lower page): forward walks take pages
// vlo + 2k, vlo + 2k + 1 (walk positions 2k, 2k + 1); backward walks vhi - 2 - 2k and
// vhi - 1 - 2k (walk positions 2k + 1, 2k).  A lane of the block-table chunk register
// holds the entry of walk position 64 c + lane.
template <int D>
__device__ __forceinline__ void step_pages(const AttnArgs& a, const SegDesc& d, int k, int bt, int npm, int len,
                                           int nring, FStep fs, bool app, PageRef& X, PageRef& Y) {
  const int vX = d.rev ? d.vhi - 2 - 2 * k : d.vlo + 2 * k;
  const int wX = d.rev ? 2 * k + 1 : 2 * k, wY = d.rev ? 2 * k : 2 * k + 1;
  X = region_a_page<D>(a, d.s, vX, wX, bt, npm, len, nring, fs, app);
  Y = region_a_page<D>(a, d.s, vX + 1, wY, bt, npm, len, nring, fs, app);
}

// Block-table entries of walk positions [64 c, 64 c + 64) of segment d (lane i: position
// 64 c + i); positions past the pool read a clamped entry that is never used.
__device__ __forceinline__ int load_bt_chunk(const AttnArgs& a, const SegDesc& d, int c) {
  const int lane = threadIdx.x & 63;
  const int w = 64 * c + lane;
  const int v = d.rev ? d.vhi - 1 - w : d.vlo + w;
  const int vv = min(max(v, 0), a.kv.max_pages_per_pair - 1);
  return a.kv.block_table[(int64_t)d.s * a.kv.max_pages_per_pair + vv];
}

// Validity bits of this lane's 8 tokens (8j .. 8j+7 of the 32-token step).
__device__ __forceinline__ uint32_t lane_valid_bits(const u32x4& rp0, const u32x4& rp1, const PageRef& X,
                                                    const PageRef& Y, int j) {
  const PageRef& P = (j < 2) ? X : Y;
  if (P.kind == 0) {
    const int n = max(0, min(8, P.nvalid - 8 * (j & 1)));
    return (1u << n) - 1u;
  }
  if (P.kind == 1) {
    uint32_t b = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b |= ((int)rp0[i] >= 0 ? 1u : 0u) << i;
      b |= ((int)rp1[i] >= 0 ? 1u : 0u) << (i + 4);
    }
    return b & ~(P.drop >> (8 * (j & 1)));
  }
  if (P.kind == 3) return (j & 1) == 0 ? 1u : 0u;
  return 0u;
}

// K fragments of a step, and the ring positions of this lane's 8 tokens (for a lane
// whose page is not a ring page the positions are read from its K page and ignored).
// Every load is unconditional, so the wait counts in the step loop stay exact.
template <int D>
__device__ __forceinline__ void load_k(const AttnArgs& a, Bf16Frags<D>& f, int pair, const PageRef& X,
                                       const PageRef& Y, int lane) {
  const int m = lane & 15, j = lane >> 4;
  // Score tile A rows: token 8*(m/4) + m%4; tile B rows: token 8*(m/4) + 4 + m%4.
  const int tA = 8 * (m >> 2) + (m & 3);
  const int tB = tA + 4;
  const PageRef& PA = (tA < 16) ? X : Y;  // tA < 16 <=> tB < 16
  const uint16_t* kbase = (PA.k != nullptr) ? PA.k : X.k;  // X is never a padding page
  const uint16_t* rowA = kbase + (tA & PA.rowmask) * D + (D / 4) * j;
  const uint16_t* rowB = kbase + (tB & PA.rowmask) * D + (D / 4) * j;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    f.kA[kk] = *reinterpret_cast<const u32x4*>(rowA + 8 * kk);
    f.kB[kk] = *reinterpret_cast<const u32x4*>(rowB + 8 * kk);
  }
  const PageRef& PT = (j < 2) ? X : Y;
  const int* pp = (PT.kind == 1)
                      ? a.ring.pos + (int64_t)pair * a.ring.window + PT.nvalid * PAGE + 8 * (j & 1)
                      : reinterpret_cast<const int*>(X.k);
  f.rp0 = *reinterpret_cast<const u32x4*>(pp);
  f.rp1 = *reinterpret_cast<const u32x4*>(pp + 4);
}

template <int D>
__device__ __forceinline__ void load_v(Bf16Frags<D>& f, const PageRef& X, const PageRef& Y, int lane) {
  const int m = lane & 15, j = lane >> 4;
  const PageRef& PV = (j < 2) ? X : Y;
  const uint16_t* vbase = (PV.v != nullptr) ? PV.v : X.v;
  // a new-token page holds V as one row [D]: the aligned 8 values containing dim 16 t + m
  // are loaded, and pv_step takes element m % 8 (unconditional loads either way)
  const bool v3 = PV.kind == 3;
  const uint16_t* vcol = vbase + (v3 ? (m & 8) : m * PAGE + 8 * (j & 1));
  const int vstride = v3 ? 16 : 16 * PAGE;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) f.v[t] = *reinterpret_cast<const u32x4*>(vcol + t * vstride);
}

template <int D>
struct SoftmaxState {
  f32x4 o[D / 16];
  float m;  // running max (log2 domain), this lane's head
  float l;  // running sum of p over this lane's tokens
};

template <int D>
__device__ __forceinline__ void state_reset(SoftmaxState<D>& st) {
#pragma unroll
  for (int t = 0; t < D / 16; ++t) st.o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = neg_inf();
  st.l = 0.f;
}

// Zero the bf16 elements of a fragment whose token bit is clear (keeps 0*garbage out
// of the MFMA when a slot of a partly filled page holds stale bits).
__device__ __forceinline__ u32x4 mask_tokens(u32x4 x, uint32_t vb) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t lo = (vb >> (2 * w)) & 1u ? 0x0000ffffu : 0u;
    uint32_t hi = (vb >> (2 * w + 1)) & 1u ? 0xffff0000u : 0u;
    r[w] = x[w] & (lo | hi);
  }
  return r;
}

template <int D>
__device__ __forceinline__ void qk_step(const Bf16Frags<D>& f, const bf16x8 (&qf)[D / 32], f32x4& sA,
                                        f32x4& sB) {
  sA = f32x4{0.f, 0.f, 0.f, 0.f};
  sB = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    sA = mfma16x16x32(as_bf16x8(f.kA[kk]), qf[kk], sA);
    sB = mfma16x16x32(as_bf16x8(f.kB[kk]), qf[kk], sB);
  }
}

// Online-softmax update for this step's 8 scores per lane; returns false when nothing
// is visible yet.  phi/plo receive the bf16 hi/lo split of the probabilities.
template <int D>
__device__ __forceinline__ bool softmax_step(const AttnArgs& a, f32x4 sA, f32x4 sB,
                                             SoftmaxState<D>& st, uint32_t vbits, bool all_valid,
                                             bf16x8& phi, bf16x8& plo) {
  float s[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = sA[i] * a.scale_log2;
    s[i + 4] = sB[i] * a.scale_log2;
  }
  if (!all_valid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = ((vbits >> i) & 1u) ? s[i] : neg_inf();
  }
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, s[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mnew = fmaxf(st.m, mx);
  if (mnew == neg_inf()) return false;  // nothing visible yet (uniform across the wave)
  const float alpha = exp2f(st.m - mnew);
  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = exp2f(s[i] - mnew);
    psum += p[i];
  }
  st.l = st.l * alpha + psum;
  st.m = mnew;
  if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) st.o[t] *= alpha;
  }
  u32x4 hi, lo;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const u32x2 hl = split_bf16x2(p[2 * w], p[2 * w + 1]);
    hi[w] = hl[0];
    lo[w] = hl[1];
  }
  phi = as_bf16x8(hi);
  plo = as_bf16x8(lo);
  return true;
}

// Element k of eight packed bf16 values, as element 0 of an otherwise zero fragment.
__device__ __forceinline__ u32x4 bf16_elem_to_front(const u32x4& x, int k) {
  const int wi = k >> 1;
  const uint32_t w = wi == 0 ? x[0] : wi == 1 ? x[1] : wi == 2 ? x[2] : x[3];
  return u32x4{(k & 1) ? (w >> 16) : (w & 0xffffu), 0u, 0u, 0u};
}

// any3: some lane's V page is a new-token page (x3 for that lane).
template <int D>
__device__ __forceinline__ void pv_step(const Bf16Frags<D>& f, SoftmaxState<D>& st, bf16x8 phi,
                                        bf16x8 plo, uint32_t vbits, bool all_valid, bool any3 = false,
                                        bool x3 = false) {
  if (any3) {
    const int m7 = threadIdx.x & 7;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const u32x4 raw = x3 ? bf16_elem_to_front(f.v[t], m7) : f.v[t];
      const bf16x8 vt = as_bf16x8(mask_tokens(raw, vbits));
      st.o[t] = mfma16x16x32(vt, phi, st.o[t]);
      st.o[t] = mfma16x16x32(vt, plo, st.o[t]);
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const bf16x8 vt = as_bf16x8(all_valid ? f.v[t] : mask_tokens(f.v[t], vbits));
    st.o[t] = mfma16x16x32(vt, phi, st.o[t]);
    st.o[t] = mfma16x16x32(vt, plo, st.o[t]);
  }
}

template <int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, int pair, bf16x8 (&qf)[D / 32]) {
  const int lane = threadIdx.x & 63, n = lane & 15, j = lane >> 4;
  const int b = pair / a.Hkv, h = pair % a.Hkv;
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.Hq + h * a.g + min(n, a.g - 1)) * D +
                      (D / 4) * j;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(q + 8 * kk);
    qf[kk] = as_bf16x8(n < a.g ? v : u32x4{0u, 0u, 0u, 0u});
  }
}

// End of a segment of `pair` whose state is in the MFMA layout (lane: head n = lane % 16,
// dims 16 t + 4 (lane / 16) + 0..3): a pair with a single record is finished here,
// otherwise the record is written for the merge kernel.
template <int D>
__device__ __forceinline__ void segment_done(const AttnArgs& a, const Plan& pl, int pair, int slot,
                                             SoftmaxState<D>& st) {
  const int lane = threadIdx.x & 63, n = lane & 15, j = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (n >= a.g) return;
  if (pair_records(pl, pair) == 1) {
    const int b = pair / a.Hkv, h = pair % a.Hkv;
    float* out = a.out + ((int64_t)b * a.Hq + h * a.g + n) * D;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) *reinterpret_cast<f32x4*>(out + 16 * t + 4 * j) = st.o[t] * inv;
    return;
  }
  float* rec = a.part + (int64_t)slot * a.rec_floats;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) *reinterpret_cast<f32x4*>(rec + n * D + 16 * t + 4 * j) = st.o[t];
  if (j == 0) {
    rec[a.g * D + n] = st.m;
    rec[a.g * D + a.g + n] = l;
  }
}

// -------------------------------------------------------------------------------
// The bf16 stream over one wave's unit of region-A pages.  One step of K/V loads is
// in flight behind the math; the next two segments are looked up ahead (one lookup per
// iteration, after the step's loads are issued), so every segment's first pages are
// addressable by the time the previous segment's last step issues their loads; the
// next pair's queries are loaded together with its first K.
// -------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void stream_a_bf16(const AttnArgs& a, const Plan& pl, const int* Lens, int u,
                                              FStep fs) {
  const int lane = threadIdx.x & 63, j = lane >> 4;
  const int nring = a.has_ring ? a.ring.window / PAGE : 0;
  UnitIter it;
  iter_init(it, pl, false, u);
  SegDesc cur = iter_next_seg(it, pl, u);
  if (!cur.ok) return;
  // Look-ahead queue: the next two segments, each valid (ok 1), past the end (ok 0) or not
  // looked up yet (ok -1).
  SegDesc nxt, nx2;
  nxt.ok = -1;
  nx2.ok = -1;
  int bt_cur0 = load_bt_chunk(a, cur, 0), bt_cur1 = 0;
  int bt_nxt = 0, bt_nx2 = 0;
  int lw = __builtin_amdgcn_readfirstlane(Lens[cur.s]);
  int len = lw & LEN_MASK;
  bool app = lw < 0;
  int npm = cdiv(len, PAGE);
  int nst = (cur.vhi - cur.vlo) >> 1;
  bool chunk_load = nst > 32;  // chunk 1 of the current segment still to request
  int cc = 0;                  // block-table chunk of the current step
  bf16x8 qf[D / 32], qn[D / 32];
  load_q<D>(a, cur.s, qf);
  PageRef x, y;
  step_pages<D>(a, cur, 0, bt_cur0, npm, len, nring, fs, app, x, y);
  Bf16Frags<D> f;
  load_k<D>(a, f, cur.s, x, y, lane);
  load_v<D>(f, x, y, lane);
  SoftmaxState<D> st;
  state_reset(st);
  int k = 0;
  for (;;) {
    const bool lastk = (k + 1 == nst);
    if (lastk && nxt.ok < 0) {
      nxt = iter_next_seg(it, pl, u);
      if (nxt.ok) bt_nxt = load_bt_chunk(a, nxt, 0);
    }
    const bool have_next = !lastk || nxt.ok > 0;
    // pages of the next step (when there is none, the current pages are loaded again,
    // which keeps every step's loads identical); the next pair's queries
    PageRef xn = x, yn = y;
    int pair_n = cur.s;
    if (!lastk) {
      const int cw = (2 * (k + 1)) >> 6;
      if (cw != cc) {
        // entering chunk cw: its entries arrived long ago; request chunk cw + 1 into the
        // register chunk cw - 1 used
        cc = cw;
        if (64 * (cc + 1) < 2 * nst) {
          if (cc & 1) bt_cur0 = load_bt_chunk(a, cur, cc + 1);
          else bt_cur1 = load_bt_chunk(a, cur, cc + 1);
        }
      }
      step_pages<D>(a, cur, k + 1, (cc & 1) ? bt_cur1 : bt_cur0, npm, len, nring, fs, app, xn, yn);
    } else if (nxt.ok > 0) {
      const int lwn = __builtin_amdgcn_readfirstlane(Lens[nxt.s]);
      const int lenn = lwn & LEN_MASK;
      step_pages<D>(a, nxt, 0, bt_nxt, cdiv(lenn, PAGE), lenn, nring, fs, lwn < 0, xn, yn);
      pair_n = nxt.s;
      load_q<D>(a, nxt.s, qn);
    }
    const uint32_t vb = lane_valid_bits(f.rp0, f.rp1, x, y, j);
    const bool allv = __ballot(vb != 0xffu) == 0;
    const bool x3 = ((j < 2) ? x.kind : y.kind) == 3;
    const bool any3 = __ballot(x3) != 0;
    f32x4 sA, sB;
    qk_step<D>(f, qf, sA, sB);
    load_k<D>(a, f, pair_n, xn, yn, lane);
    bf16x8 phi, plo;
    if (softmax_step<D>(a, sA, sB, st, vb, allv, phi, plo)) pv_step<D>(f, st, phi, plo, vb, allv, any3, x3);
    load_v<D>(f, xn, yn, lane);
    if (lastk) {
      segment_done<D>(a, pl, cur.s, slot_of(pl, cur), st);
      state_reset(st);
    }
    // look-ahead requests (rare), at most one lookup per iteration
    if (chunk_load) {
      bt_cur1 = load_bt_chunk(a, cur, 1);
      chunk_load = false;
    }
    if (nxt.ok < 0) {
      nxt = iter_next_seg(it, pl, u);
      if (nxt.ok) bt_nxt = load_bt_chunk(a, nxt, 0);
    } else if (nxt.ok > 0 && nx2.ok < 0) {
      nx2 = iter_next_seg(it, pl, u);
      if (nx2.ok) bt_nx2 = load_bt_chunk(a, nx2, 0);
    }
    if (!have_next) break;
    x = xn;
    y = yn;
    if (lastk) {
      cur = nxt;
      nxt = nx2;
      bt_cur0 = bt_nxt;
      bt_nxt = bt_nx2;
      lw = __builtin_amdgcn_readfirstlane(Lens[cur.s]);
      len = lw & LEN_MASK;
      app = lw < 0;
      npm = cdiv(len, PAGE);
      nst = (cur.vhi - cur.vlo) >> 1;
      chunk_load = nst > 32;
      cc = 0;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qf[kk] = qn[kk];
      nx2.ok = -1;
      k = 0;
    } else {
      ++k;
    }
  }
}

// -------------------------------------------------------------------------------
// Low-precision region (BeaconKV demoted tokens, int8 or int4 codes): codes -> bf16
// exactly, per-token scales.
// -------------------------------------------------------------------------------
// Two fp32 values whose low 16 bits are zero (small integers) -> packed bf16x2, in
// one byte permute (bytes 2-3 of lo, then bytes 2-3 of hi).
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

__device__ __forceinline__ uint32_t i8pair_to_bf16x2(uint32_t word, int byte0) {
  const float f0 = (float)(int)(int8_t)((word >> (8 * byte0)) & 0xffu);
  const float f1 = (float)(int)(int8_t)((word >> (8 * (byte0 + 1))) & 0xffu);
  return pack_hi16(f0, f1);
}

// 8 int8 codes (two dwords) -> 8 bf16 (exact: |code| <= 127).
__device__ __forceinline__ u32x4 i8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = i8pair_to_bf16x2(w0, 0);
  r[1] = i8pair_to_bf16x2(w0, 2);
  r[2] = i8pair_to_bf16x2(w1, 0);
  r[3] = i8pair_to_bf16x2(w1, 2);
  return r;
}

// 8 int4 codes (one dword, element e in nibble e, two's complement) -> 8 bf16 holding
// I4_OFFSET + code, exactly.  Flipping each nibble's sign bit gives the offset-binary
// code u = code + 8 in 0..15; bf16 0x4300 | u is 2^7 (1 + u / 128) = 128 + u, so a
// byte permute that spreads the nibbles into the low mantissa bytes plus one OR with
// the exponent decodes two elements.  The offset is taken out after the MFMAs: of the
// scores as I4_OFFSET * sum_k q_k per head, of the outputs as I4_OFFSET * sum_t p_t.
constexpr float I4_OFFSET = 136.0f;
__device__ __forceinline__ u32x4 i4x8_to_bf16x8(uint32_t w) {
  const uint32_t u = w ^ 0x88888888u;
  const uint32_t lo = u & 0x0f0f0f0fu;         // elements 0, 2, 4, 6 in bytes 0..3
  const uint32_t hi = (u >> 4) & 0x0f0f0f0fu;  // elements 1, 3, 5, 7
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q)  // byte 0 <- lo byte q, byte 2 <- hi byte q, bytes 1 and 3 zero
    r[q] = __builtin_amdgcn_perm(hi, lo, 0x0c000c00u | ((4u + q) << 16) | q) | 0x43004300u;
  return r;
}

// 8 E4M3 codes (two dwords, element e in byte e) -> 8 bf16, exactly.  A normal code
// (exponent field e >= 1) is 2^(e - 7) (1 + m / 8), whose bf16 pattern is the code's 7
// low bits shifted left by 4 plus (127 - 7) << 7, the sign moved to bit 15: two per
// dword after a byte permute.  Exponent field 0 (zero, and the subnormals m 2^-9) is
// rare after absmax scaling; a fragment holding one in any lane decodes element by
// element.  The NaN codes decode as 480 (finite), like the other codes of unused slots,
// whose weights are exactly zero.
struct F8x8 {
  u32x2 w;
};
__device__ __forceinline__ uint32_t f8_code_to_bf16(uint32_t c) {
  const uint32_t c7 = c & 0x7fu;
  uint32_t v;
  if (c7 >= 8u) {
    v = (c7 << 4) + 0x3C00u;
  } else if (c7 == 0u) {
    v = 0u;
  } else {  // m 2^-9 = 2^(e - 9) (m / 2^e) with e = floor(log2 m)
    const uint32_t e = 31u - __builtin_clz(c7);
    v = ((118u + e) << 7) | ((c7 << (7u - e)) & 0x7fu);
  }
  return v | ((c & 0x80u) << 8);
}
__device__ __forceinline__ u32x4 f8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const uint32_t small = (~((w0 & 0x7f7f7f7fu) + 0x78787878u) | ~((w1 & 0x7f7f7f7fu) + 0x78787878u)) &
                         0x80808080u;  // bit 7 of a byte: that code's 7 low bits are < 8
  u32x4 r;
  if (__builtin_expect(__ballot(small != 0u) != 0, 0)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = q < 2 ? w0 : w1, sh = 16u * (q & 1);
      r[q] = f8_code_to_bf16((w >> sh) & 0xffu) | (f8_code_to_bf16((w >> (sh + 8)) & 0xffu) << 16);
    }
    return r;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t w = i ? w1 : w0;
    const uint32_t c7 = w & 0x7f7f7f7fu, sg = w & 0x80808080u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // codes 2h, 2h + 1 of the dword -> bits 0..15, 16..31
      const uint32_t sel = h ? 0x0c030c02u : 0x0c010c00u;
      r[2 * i + h] = ((__builtin_amdgcn_perm(0u, c7, sel) << 4) + 0x3C003C00u) |
                     (__builtin_amdgcn_perm(0u, sg, sel) << 8);
    }
  }
  return r;
}

// 8 codes of a fragment: two dwords of int8 or fp8 codes, or one dword of int4 codes.
template <int BITS, bool F8 = false> struct LpWord { typedef u32x2 T; };
template <> struct LpWord<4, false> { typedef uint32_t T; };
template <> struct LpWord<8, true> { typedef F8x8 T; };
__device__ __forceinline__ u32x4 lp_to_bf16x8(u32x2 w) { return i8x8_to_bf16x8(w[0], w[1]); }
__device__ __forceinline__ u32x4 lp_to_bf16x8(uint32_t w) { return i4x8_to_bf16x8(w); }
__device__ __forceinline__ u32x4 lp_to_bf16x8(F8x8 x) { return f8x8_to_bf16x8(x.w[0], x.w[1]); }

template <int D, int BITS, bool F8 = false>
struct LpFrags {
  typedef typename LpWord<BITS, F8>::T W;
  W kA[D / 32];  // 8 K codes per MFMA K-step, score tile A row
  W kB[D / 32];
  W v[D / 16];   // 8 V^T codes per output tile
  f32x4 ks[2];   // K scales of this lane's 8 tokens
  f32x4 vs[2];   // V scales of this lane's 8 tokens
};

// Byte offsets scale with the code width: a K row is D * BITS / 8 bytes, a V^T row
// 16 * BITS / 8.
template <int D, int BITS, bool F8>
__device__ __forceinline__ void load_lp_k(const AttnArgs& a, LpFrags<D, BITS, F8>& f, int pgX, int pgY, int lane) {
  typedef typename LpWord<BITS, F8>::T W;
  const int m = lane & 15, j = lane >> 4;
  const int tA = 8 * (m >> 2) + (m & 3), tB = tA + 4;
  const int pgK = (tA < 16) ? pgX : pgY;
  const int8_t* kbase = a.kv.k8_pages + (int64_t)pgK * PAGE * D * BITS / 8;
  const int8_t* rowA = kbase + ((tA & 15) * D + (D / 4) * j) * BITS / 8;
  const int8_t* rowB = kbase + ((tB & 15) * D + (D / 4) * j) * BITS / 8;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    f.kA[kk] = *reinterpret_cast<const W*>(rowA + kk * BITS);
    f.kB[kk] = *reinterpret_cast<const W*>(rowB + kk * BITS);
  }
  const int pgT = (j < 2) ? pgX : pgY;
  const float* ksc = a.kv.k8_scale + (int64_t)pgT * PAGE + 8 * (j & 1);
  f.ks[0] = *reinterpret_cast<const f32x4*>(ksc);
  f.ks[1] = *reinterpret_cast<const f32x4*>(ksc + 4);
}

template <int D, int BITS, bool F8>
__device__ __forceinline__ void load_lp_v(const AttnArgs& a, LpFrags<D, BITS, F8>& f, int pgX, int pgY, int lane) {
  typedef typename LpWord<BITS, F8>::T W;
  const int m = lane & 15, j = lane >> 4;
  const int pgT = (j < 2) ? pgX : pgY;
  const int8_t* vcol = a.kv.v8_pages + ((int64_t)pgT * PAGE * D + m * PAGE + 8 * (j & 1)) * BITS / 8;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) f.v[t] = *reinterpret_cast<const W*>(vcol + t * 16 * PAGE * BITS / 8);
  const float* vsc = a.kv.v8_scale + (int64_t)pgT * PAGE + 8 * (j & 1);
  f.vs[0] = *reinterpret_cast<const f32x4*>(vsc);
  f.vs[1] = *reinterpret_cast<const f32x4*>(vsc + 4);
}

template <int D, int BITS, int NSET, bool F8 = false>
__device__ __forceinline__ void run_region_b_lp(const AttnArgs& a, int pair, int v0, int v1, bool rev, SoftmaxState<D>& st) {
  static_assert(NSET % 2 == 0, "steps are folded in pairs");
  const int lane = threadIdx.x & 63, j = lane >> 4;
  bf16x8 qf[D / 32];
  load_q<D>(a, pair, qf);
  state_reset(st);
  // int4: I4_OFFSET * (sum of this lane's head's query) comes off every score; psum is
  // one more output tile, sum_t p_t per head, accumulated by MFMA from the same bf16
  // weights as the outputs (a ones operand in place of V) and rescaled with them, so
  // I4_OFFSET * psum is exactly the offset the decoded V values added
  float qoff = 0.f;
  f32x4 psum = {0.f, 0.f, 0.f, 0.f};
  if constexpr (BITS == 4) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const u32x4 w = __builtin_bit_cast(u32x4, qf[kk]);
#pragma unroll
      for (int e = 0; e < 4; ++e) qoff += bf16_to_f32(w[e] & 0xffffu) + bf16_to_f32(w[e] >> 16);
    }
    qoff += __shfl_xor(qoff, 16);
    qoff += __shfl_xor(qoff, 32);
    qoff *= I4_OFFSET;
  }
  const int len = __builtin_amdgcn_readfirstlane(a.kv.length8[pair]);
  const int npm = cdiv(len, PAGE);  // v1 <= npm rounded up to even; the pad page is never loaded
  const int nch = (v1 - v0 + 63) / 64;
  for (int ci = 0; ci < nch; ++ci) {
    const int c0 = v0 + 64 * (rev ? nch - 1 - ci : ci);
    const int c1 = min(v1, c0 + 64);
    int bt = 0;
    if (c0 + lane < min(c1, npm))
      bt = a.kv.block_table8[(int64_t)pair * a.kv.max_pages8_per_pair + c0 + lane];
    auto page = [&](int vp) -> int {
      // the pad page of an odd page count re-uses the previous page (all slots masked)
      return __builtin_amdgcn_readlane(bt, min(vp, npm - 1) - c0);
    };
    // NSET steps of loads in flight, and steps folded in pairs (64 tokens) into one
    // online-softmax update.  A step here moves half (int8) or a quarter (int4) of a
    // bf16 step's bytes, so with one step in flight per wave the whole device would hold
    // too few bytes in flight to cover the memory latency (measured: the int4 pool ran
    // at the same step rate as int8, half the bandwidth).  A set is refilled with the
    // step NSET ahead right after its last use (K after the QK MFMAs, V after the PV
    // MFMAs).  Steps past the end of the range run on a repeat of the last pages with
    // every token masked, and their refills repeat the last pages too, so every block
    // issues the same loads and the wait counts stay exact.
    const int nst = (c1 - c0) / 2;
    auto vat = [&](int i) {
      i = min(i, nst - 1);
      return c0 + 2 * (rev ? nst - 1 - i : i);
    };
    auto valid_bits = [&](int v, bool real) -> uint32_t {
      const int nvT = real ? max(0, min(PAGE, len - (v + (j >> 1)) * PAGE)) : 0;
      return (uint32_t)((1 << max(0, min(8, nvT - 8 * (j & 1)))) - 1);
    };
    auto qk = [&](const LpFrags<D, BITS, F8>& f, float (&s)[8], float (&vsc)[8]) {
      f32x4 sA = {0.f, 0.f, 0.f, 0.f}, sB = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        sA = mfma16x16x32(as_bf16x8(lp_to_bf16x8(f.kA[kk])), qf[kk], sA);
        sB = mfma16x16x32(as_bf16x8(lp_to_bf16x8(f.kB[kk])), qf[kk], sB);
      }
      if constexpr (BITS == 4) {
        sA -= qoff;
        sB -= qoff;
      }
      // per-token K scale folds into the logits; V scale into the probabilities
      sA = sA * f.ks[0];
      sB = sB * f.ks[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = sA[i] * a.scale_log2;
        s[i + 4] = sB[i] * a.scale_log2;
        vsc[i] = f.vs[0][i];
        vsc[i + 4] = f.vs[1][i];
      }
    };
    auto mask = [&](float (&s)[8], float (&vsc)[8], uint32_t vb) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = (vb >> i) & 1u;
        s[i] = ok ? s[i] : neg_inf();
        vsc[i] = ok ? vsc[i] : 0.f;
      }
    };
    // sum_t p_t (scale_t code_t) = sum_t (p_t scale_t) code_t, weights split bf16 hi + lo
    auto pv = [&](const LpFrags<D, BITS, F8>& f, const float (&p)[8], const float (&vsc)[8]) {
      u32x4 hi, lo;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 hl = split_bf16x2(p[2 * w] * vsc[2 * w], p[2 * w + 1] * vsc[2 * w + 1]);
        hi[w] = hl[0];
        lo[w] = hl[1];
      }
      const bf16x8 phi = as_bf16x8(hi), plo = as_bf16x8(lo);
      if constexpr (BITS == 4) {
        const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
        psum = mfma16x16x32(ones, phi, psum);
        psum = mfma16x16x32(ones, plo, psum);
      }
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        // every code decodes to a finite value and the weight of an unused slot is
        // exactly 0, so unlike the bf16 pool (whose unused slots may hold NaN bits) no
        // element needs zeroing
        const u32x4 vt = lp_to_bf16x8(f.v[t]);
        st.o[t] = mfma16x16x32(as_bf16x8(vt), phi, st.o[t]);
        st.o[t] = mfma16x16x32(as_bf16x8(vt), plo, st.o[t]);
      }
    };
    // NSET register sets in a ring: set r holds step i + r of the block being worked on
    // and is refilled with step i + r + NSET right after its last use.
    LpFrags<D, BITS, F8> f[NSET];
#pragma unroll
    for (int r = 0; r < NSET; ++r) {
      load_lp_k<D, BITS, F8>(a, f[r], page(vat(r)), page(vat(r) + 1), lane);
      load_lp_v<D, BITS, F8>(a, f[r], page(vat(r)), page(vat(r) + 1), lane);
    }
    for (int i = 0; i < nst; i += NSET) {
#pragma unroll
      for (int r = 0; r < NSET; r += 2) {
        const int va = vat(i + r), vb_ = vat(i + r + 1);
        const int vna = vat(i + r + NSET), vnb = vat(i + r + 1 + NSET);
        const uint32_t m0 = valid_bits(va, i + r < nst), m1 = valid_bits(vb_, i + r + 1 < nst);
        const bool allv = __ballot((m0 & m1) != 0xffu) == 0;
        float s0[8], s1[8], c0s[8], c1s[8];
        qk(f[r], s0, c0s);
        qk(f[r + 1], s1, c1s);
        load_lp_k<D, BITS, F8>(a, f[r], page(vna), page(vna + 1), lane);
        load_lp_k<D, BITS, F8>(a, f[r + 1], page(vnb), page(vnb + 1), lane);
        if (!allv) {
          mask(s0, c0s, m0);
          mask(s1, c1s, m1);
        }
        float mx = s0[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s0[e]);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, s1[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(st.m, mx);
        if (mnew != neg_inf()) {
          const float alpha = exp2f(st.m - mnew);
          float p0[8], p1[8], ps = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p0[e] = exp2f(s0[e] - mnew);
            p1[e] = exp2f(s1[e] - mnew);
            ps += p0[e] + p1[e];
          }
          st.l = st.l * alpha + ps;
          st.m = mnew;
          if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
            for (int t = 0; t < D / 16; ++t) st.o[t] *= alpha;
            if constexpr (BITS == 4) psum *= alpha;
          }
          pv(f[r], p0, c0s);
          pv(f[r + 1], p1, c1s);
        }
        load_lp_v<D, BITS, F8>(a, f[r], page(vna), page(vna + 1), lane);
        load_lp_v<D, BITS, F8>(a, f[r + 1], page(vnb), page(vnb + 1), lane);
      }
    }
  }
  if constexpr (BITS == 4) {
    const float off = I4_OFFSET * psum[0];  // every row of the tile holds the same sum
#pragma unroll
    for (int t = 0; t < D / 16; ++t) st.o[t] -= off;
  }
}

// -------------------------------------------------------------------------------
// fp32 region A (VALU; small head dims / tiny workloads)
// -------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void run_region_a_f32(const AttnArgs& a, const Plan& pl, int pair, int v0, int v1,
                                                 int slot, float* wlds) {
  // wlds: this wave's LDS area: q [16][D] then p [16][32]
  const int lane = threadIdx.x & 63;
  const int g = a.g;
  const int b = pair / a.Hkv, h = pair % a.Hkv;
  float* qs = wlds;
  float* ps = wlds + 16 * D;
  const float* q = reinterpret_cast<const float*>(a.q) + ((int64_t)b * a.Hq + h * g) * D;
  for (int i = lane; i < g * D; i += 64) qs[i] = q[i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  float mrun[16], lrun[16];
  float o[16][D / 64 > 0 ? D / 64 : 1];
  for (int n = 0; n < 16; ++n) {
    mrun[n] = neg_inf();
    lrun[n] = 0.f;
    for (int e = 0; e < D / 64; ++e) o[n][e] = 0.f;
  }
  const int len = a.kv.length[pair];
  const int npm = cdiv(len, PAGE);
  const int nring = a.has_ring ? a.ring.window / PAGE : 0;
  const int tok = lane & 31, half = lane >> 5;
  for (int v = v0; v < v1; v += 2) {
    const float* kp[2];
    const float* vp[2];
    int nvalid[2];
    int ringp[2];
    for (int u = 0; u < 2; ++u) {
      int vv = v + u;
      kp[u] = nullptr;
      vp[u] = nullptr;
      nvalid[u] = 0;
      ringp[u] = -1;
      if (vv < npm) {
        int pg = a.kv.block_table[(int64_t)pair * a.kv.max_pages_per_pair + vv];
        kp[u] = reinterpret_cast<const float*>(a.kv.k_pages) + (int64_t)pg * PAGE * D;
        vp[u] = reinterpret_cast<const float*>(a.kv.v_pages) + (int64_t)pg * PAGE * D;
        nvalid[u] = min(PAGE, len - vv * PAGE);
      } else if (vv < npm + nring) {
        int rp = vv - npm;
        int64_t off = ((int64_t)pair * nring + rp) * PAGE * D;
        kp[u] = reinterpret_cast<const float*>(a.ring.k) + off;
        vp[u] = reinterpret_cast<const float*>(a.ring.v) + off;
        ringp[u] = rp;
      }
    }
    // validity of token `tok` (and of every token, for the PV loop below)
    auto valid_of = [&](int t) -> bool {
      int u = t >> 4, sl = t & 15;
      if (kp[u] == nullptr) return false;
      if (ringp[u] < 0) return sl < nvalid[u];
      return a.ring.pos[(int64_t)pair * a.ring.window + ringp[u] * PAGE + sl] >= 0;
    };
    const bool myvalid = valid_of(tok);
    float sc[16];
    for (int n = 0; n < 16; ++n) sc[n] = 0.f;
    if (myvalid) {
      const float* krow = kp[tok >> 4] + (tok & 15) * D + half * (D / 2);
      for (int d = 0; d < D / 2; ++d) {
        float kv = krow[d];
        for (int n = 0; n < g; ++n) sc[n] += kv * qs[n * D + half * (D / 2) + d];
      }
    }
    for (int n = 0; n < g; ++n) {
      float s = sc[n] + __shfl_xor(sc[n], 32);
      s = myvalid ? s * a.scale_log2 : neg_inf();
      float mx = wave_max(s);
      float mnew = fmaxf(mrun[n], mx);
      float p = (mnew == neg_inf()) ? 0.f : exp2f(s - mnew);
      float alpha = (mnew == neg_inf()) ? 1.f : exp2f(mrun[n] - mnew);
      float psum = p;
      for (int off = 16; off > 0; off >>= 1) psum += __shfl_xor(psum, off);  // within 32 lanes
      lrun[n] = lrun[n] * alpha + psum;
      mrun[n] = mnew;
      for (int e = 0; e < D / 64; ++e) o[n][e] *= alpha;
      if (half == 0) ps[n * 32 + tok] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    for (int t = 0; t < 32; ++t) {
      int u = t >> 4, sl = t & 15;
      if (!valid_of(t)) continue;
      for (int e = 0; e < D / 64; ++e) {
        int d = lane + 64 * e;
        float vv = vp[u][d * PAGE + sl];
        for (int n = 0; n < g; ++n) o[n][e] += ps[n * 32 + t] * vv;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  // end of the segment: a pair with a single record is finished here, else the record is
  // written for the merge kernel
  float* out = a.out + ((int64_t)b * a.Hq + h * g) * D;
  if (pair_records(pl, pair) == 1) {
    for (int n = 0; n < g; ++n) {
      const float inv = lrun[n] > 0.f ? 1.0f / lrun[n] : 0.f;
      for (int e = 0; e < D / 64; ++e) out[n * D + lane + 64 * e] = o[n][e] * inv;
    }
    return;
  }
  float* rec = a.part + (int64_t)slot * a.rec_floats;
  for (int n = 0; n < g; ++n) {
    for (int e = 0; e < D / 64; ++e) rec[n * D + lane + 64 * e] = o[n][e];
    if (lane == 0) {
      rec[g * D + n] = mrun[n];
      rec[g * D + g + n] = lrun[n];
    }
  }
}

// Region-B (low-precision) and fp32 segments: one segment at a time (its query, length
// and block table fetched at its start).
template <int D, bool F32, int BITS, bool F8 = false>
__device__ __forceinline__ void stream_segments(const AttnArgs& a, const Plan& pl, bool seqB, int u, float* wlds) {
  UnitIter it;
  iter_init(it, pl, seqB, u);
  const int np = pl.np;
  for (;;) {
    const SegDesc d = iter_next_seg(it, pl, u);
    if (!d.ok) break;
    if constexpr (F32) {
      run_region_a_f32<D>(a, pl, d.s, d.vlo, d.vhi, slot_of(pl, d), wlds);
    } else {
      SoftmaxState<D> st;
      run_region_b_lp<D, BITS, ATTN_LP_SETS, F8>(a, d.s - np, d.vlo, d.vhi, d.rev != 0, st);
      segment_done<D>(a, pl, d.s - np, slot_of(pl, d), st);
    }
  }
}

// -------------------------------------------------------------------------------
// The streaming kernel
// -------------------------------------------------------------------------------
// WPE work-groups per CU (ATTN_GRID * WPE of them): with WPE = 1 a wave may use a whole
// SIMD's registers; with WPE = 2 (int4 pools) each wave fits in half of them.
// LP: the cache has a low-precision pool; the instantiation without one keeps the
// code-pool path's register needs out of the bf16 loop's allocation.
template <int D, bool F32, bool LP, int WPE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void decode_attn_kernel(AttnArgs a) {
  extern __shared__ int lds[];
  const int np = a.kv.num_pairs;
  const int nseg = plan_regions(a);
  int* P = a.gplan ? a.plan : lds;
  int* Lens = a.gplan ? a.plan + nseg + 2 : lds + nseg + 1;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // fused step: the position being appended and the ring slot it turns over
  FStep fs{-1, 0};
  int p = 0;
  float tau = 0.f;
  if (a.fstep) {
    p = a.st.pos_dev[0];
    tau = a.st.tau_dev[0];
    const int slot = ((p % a.ring.window) + a.ring.window) % a.ring.window;
    fs.rp = slot / PAGE;
    fs.rs = slot % PAGE;
  }
  __shared__ int wsum[ATTN_WG_WAVES];
  if (a.gplan) {
    // the plan kernel wrote the plan; every wave may take first-layer slices
    if constexpr (!F32 && !LP) {
      if (a.fgemm) small_gemm_slices(a.gm, blockIdx.x * ATTN_WG_WAVES + wid, gridDim.x * ATTN_WG_WAVES);
    }
  } else if (a.fgemm) {
    // wave 0 builds the plan while the other waves take first-layer slices
    if (wid == 0) compute_plan(a, P, Lens, nseg, fs.rp * PAGE + fs.rs, tau);
    else if constexpr (!F32 && !LP)
      small_gemm_slices(a.gm, blockIdx.x * (ATTN_WG_WAVES - 1) + wid - 1, gridDim.x * (ATTN_WG_WAVES - 1));
  } else {
    compute_plan_wg<ATTN_WG_WAVES * 64>(a, P, Lens, nseg, fs.rp * PAGE + fs.rs, tau, wsum);
  }
  __syncthreads();
  // the merge kernel reads the prefix (and the position) from here
  if (!a.gplan && blockIdx.x == 0) {
    for (int s = threadIdx.x; s <= nseg; s += blockDim.x) a.plan[s] = P[s];
    if (threadIdx.x == 0) a.plan[nseg + 1] = p;
  }
  // Work-groups are dispatched round-robin over the 8 XCDs; numbering the units so that
  // each XCD takes one contiguous eighth of a sequence evens out the XCDs' finish times
  // (measured: 1-3 us at the 361 MB and 543 MB caches).
  const int gw = ((blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8) * ATTN_WG_WAVES + wid;
  const Plan pl = make_plan(P, np, gridDim.x * ATTN_WG_WAVES, LP);
  float* wlds = nullptr;
  if constexpr (F32) wlds = reinterpret_cast<float*>(lds + (a.gplan ? 0 : 2 * nseg + 2)) + wid * (16 * D + 16 * 32);
  if constexpr (F32) {
    stream_segments<D, true, 8>(a, pl, false, gw, wlds);
  } else {
    stream_a_bf16<D>(a, pl, Lens, gw, fs);
    if constexpr (LP) {
      if (a.kv.lp_bits == KVP_LP_INT4) stream_segments<D, false, 4>(a, pl, true, gw, nullptr);
      else if (a.kv.lp_bits == KVP_LP_FP8_E4M3) stream_segments<D, false, 8, true>(a, pl, true, gw, nullptr);
      else stream_segments<D, false, 8>(a, pl, true, gw, nullptr);
    }
  }
}

// -------------------------------------------------------------------------------
// Plan for caches whose P and Lens would not fit in LDS: one work-group computes them into
// the workspace (and, for a fused step, the position the merge kernel applies), before
// the stream kernel, whose waves then read them from global memory.
// -------------------------------------------------------------------------------
constexpr int PLAN_THREADS = 1024;
__global__ __launch_bounds__(PLAN_THREADS) void decode_attn_plan_kernel(AttnArgs a) {
  __shared__ int wsum[PLAN_THREADS / 64];
  const int nseg = plan_regions(a);
  int slot = 0, p = 0;
  float tau = 0.f;
  if (a.fstep) {
    p = a.st.pos_dev[0];
    tau = a.st.tau_dev[0];
    slot = ((p % a.ring.window) + a.ring.window) % a.ring.window;
  }
  compute_plan_wg<PLAN_THREADS>(a, a.plan, a.plan + nseg + 2, nseg, slot, tau, wsum);
  if (threadIdx.x == 0) a.plan[nseg + 1] = p;
}

// -------------------------------------------------------------------------------
// Merge: one wave per (pair, query head).  The pair's records are the segments of its
// A region then of its B region, consecutive slots each; the wave requests the (m, l)
// of the first 64 records (one per lane) and the outputs of the first 16 in one batch,
// so a pair with up to 16 records costs two memory round trips.  The reference max M
// covers every record; the normaliser is sum_k 2^(m_k - M) l_k and the output
// sum_k 2^(m_k - M) o_k / normaliser, accumulated in record order, so the result is
// deterministic.  A pair with no visible token gets zeros; a pair with a single record
// was finished by the streaming kernel.
// -------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_attn_merge_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int np = a.kv.num_pairs, g = a.g;
  if (a.fstep && w >= np * g && w < np * (g + 1)) {
    // fused step: waves np g .. np (g + 1) - 1 apply the delayed step of one pair each,
    // now that every read of the ring slots is done; their memory round trips overlap
    // the merge waves'
    const int pair = w - np * g;
    const int p = a.plan[np + 1];
    step_pair<uint16_t, D>(a.st, pair, p);
    if (pair == 0 && lane == 0) a.st.pos_dev[0] = p + 1;
    return;
  }
  if (w >= np * g) return;
  const int pair = w / g, n = w % g;
  const Plan pl = make_plan(a.plan, np, a.nw, a.kv.num_pages8 > 0);
  int ufA = 0, ufB = 0;
  const int na = region_records(pl, pair, ufA);
  const int nb = pl.lp ? region_records(pl, np + pair, ufB) : 0;
  const int nrec = na + nb;
  const int b = pair / a.Hkv, h = pair % a.Hkv;
  float* out = a.out + ((int64_t)b * a.Hq + h * g + n) * D;
  if (nrec == 1) return;
  if (nrec == 0) {
#pragma unroll
    for (int e = 0; e < D / 64; ++e) out[lane + 64 * e] = 0.f;
    return;
  }
  const int r0 = pair + ufA, s0 = pl.baseB + pair + ufB;
  auto rec = [&](int k) {
    const int slot = (k < na) ? r0 + k : s0 + (k - na);
    return a.part + (int64_t)slot * a.rec_floats;
  };
  // first batch: lane k < 64 holds record k's (m, l); outputs of records 0..15
  const float* rl = rec(min(lane, nrec - 1));
  float m0 = rl[g * D + n], l0 = rl[g * D + g + n];
  float ov0[16][D / 64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float* o = rec(min(i, nrec - 1)) + n * D;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) ov0[i][e] = o[lane + 64 * e];
  }
  if (lane >= nrec) {
    m0 = neg_inf();
    l0 = 0.f;
  }
  float M = m0;
  for (int k = lane + 64; k < nrec; k += 64) M = fmaxf(M, rec(k)[g * D + n]);
  M = wave_max(M);
  float acc[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
  float den = 0.f;
  if (M != neg_inf()) {
    for (int k0 = 0; k0 < nrec; k0 += 64) {
      const int k = k0 + lane;
      float wk = 0.f, lk = 0.f;
      if (k0 == 0) {
        wk = (m0 == neg_inf()) ? 0.f : exp2f(m0 - M);
        lk = l0;
      } else if (k < nrec) {
        const float m = rec(k)[g * D + n];
        wk = (m == neg_inf()) ? 0.f : exp2f(m - M);
        lk = rec(k)[g * D + g + n];
      }
      den += wk * lk;
      const int kn = min(64, nrec - k0);
      // batches of 16 records: all loads issued before the accumulation
      for (int kb = 0; kb < kn; kb += 16) {
        float ov[16][D / 64];
        if (k0 == 0 && kb == 0) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int e = 0; e < D / 64; ++e) ov[i][e] = ov0[i][e];
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kk = min(kb + i, kn - 1);
            const float* o = rec(k0 + kk) + n * D;
#pragma unroll
            for (int e = 0; e < D / 64; ++e) ov[i][e] = o[lane + 64 * e];
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float wb = (kb + i < kn) ? __shfl(wk, kb + i) : 0.f;
#pragma unroll
          for (int e = 0; e < D / 64; ++e) acc[e] += wb * ov[i][e];
        }
      }
    }
    den = wave_sum(den);
  }
  const float inv = (den > 0.f) ? 1.0f / den : 0.f;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) out[lane + 64 * e] = acc[e] * inv;
}

// LDS: page prefix P[nseg + 1], the pool lengths [num_pairs] (padded to nseg + 1 ints),
// and for fp32 caches one scratch area per wave.
size_t attn_lds_bytes(int num_pairs, int D, bool f32, bool lp) {
  const size_t nseg = (size_t)(lp ? 2 : 1) * num_pairs;
  size_t b = 2 * (nseg + 1) * sizeof(int);
  if (f32) b += (size_t)ATTN_WG_WAVES * (16 * D + 16 * 32) * sizeof(float);
  return b;
}

}  // namespace kvp

using namespace kvp;

// Workspace: [plan: 2 num_pairs + 1 ints][records].  Record slots: per sequence, regions
// + units (every segment is one (region, unit) pair and s + u is unique), for the
// largest launch (two waves per SIMD).
// Plan area: P[0..nseg] (nseg <= 2 num_pairs), the position, and Lens[num_pairs] when the
// plan lives in global memory.
static size_t attn_plan_bytes(int num_pairs) { return (((size_t)(3 * num_pairs + 2) * sizeof(int)) + 255) & ~(size_t)255; }
static size_t attn_rec_floats(int g, int D) { return ((size_t)g * (D + 2) + 3) & ~(size_t)3; }
static size_t attn_max_slots(int num_pairs) { return 2 * ((size_t)num_pairs + ATTN_MAX_NWAVES); }

extern "C" size_t kvp_decode_attn_workspace_size(int32_t B, int32_t Hq, int32_t num_pairs,
                                                 int32_t head_dim) {
  if (B <= 0 || Hq <= 0 || num_pairs <= 0 || head_dim <= 0 || num_pairs % B != 0) return 0;
  const int Hkv = num_pairs / B;
  if (Hq % Hkv != 0) return 0;
  const int g = Hq / Hkv;
  return attn_plan_bytes(num_pairs) + attn_max_slots(num_pairs) * attn_rec_floats(g, head_dim) * sizeof(float);
}

static kvp_status launch_attn(const void* q, int B, int Hq, const kvp_paged_kv* kv, const kvp_ring* ring,
                              float sm_scale, float* out, void* ws, hipStream_t stream,
                              const StepArgs* fused, const SmallGemm* gm = nullptr) {
  AttnArgs a;
  a.fstep = fused != nullptr;
  if (fused) a.st = *fused;
  a.fgemm = gm != nullptr;
  if (gm) a.gm = *gm;
  a.q = q;
  a.out = out;
  a.B = B;
  a.Hkv = kv->num_pairs / B;
  a.Hq = Hq;
  a.g = Hq / a.Hkv;
  a.D = kv->head_dim;
  a.kv = *kv;
  a.has_ring = ring != nullptr;
  if (ring) a.ring = *ring;
  else a.ring = kvp_ring{};
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.plan = reinterpret_cast<int*>(ws);
  a.part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + attn_plan_bytes(kv->num_pairs));
  a.rec_floats = (int)attn_rec_floats(a.g, a.D);
  const bool f32 = kv->dtype == KVP_F32;
  const bool lp = kv->num_pages8 > 0;
  size_t lds = attn_lds_bytes(kv->num_pairs, a.D, f32, lp);
  a.gplan = lds > 160 * 1024 - 64;  // room for the kernel's static LDS
  if (a.gplan) {
    lds = attn_lds_bytes(0, a.D, f32, lp) - 2 * sizeof(int);  // no plan in LDS
    hipLaunchKernelGGL(decode_attn_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, a);
    KVP_LAUNCH_CHECK();
  }
  const dim3 g1(ATTN_GRID), g2(ATTN_GRID * 2), b(256);
  a.nw = ATTN_GRID * ATTN_WG_WAVES;
  if (f32) {
    if (a.D == 64) hipLaunchKernelGGL((decode_attn_kernel<64, true, false, 1>), g1, b, lds, stream, a);
    else hipLaunchKernelGGL((decode_attn_kernel<128, true, false, 1>), g1, b, lds, stream, a);
  } else if (lp && (kv->lp_bits == KVP_LP_INT4 || kv->lp_bits == KVP_LP_FP8_E4M3)) {
    a.nw = 2 * ATTN_GRID * ATTN_WG_WAVES;
    if (a.D == 64) hipLaunchKernelGGL((decode_attn_kernel<64, false, true, 2>), g2, b, lds, stream, a);
    else hipLaunchKernelGGL((decode_attn_kernel<128, false, true, 2>), g2, b, lds, stream, a);
  } else if (lp) {
    if (a.D == 64) hipLaunchKernelGGL((decode_attn_kernel<64, false, true, 1>), g1, b, lds, stream, a);
    else hipLaunchKernelGGL((decode_attn_kernel<128, false, true, 1>), g1, b, lds, stream, a);
  } else {
    if (a.D == 64) hipLaunchKernelGGL((decode_attn_kernel<64, false, false, 1>), g1, b, lds, stream, a);
    else hipLaunchKernelGGL((decode_attn_kernel<128, false, false, 1>), g1, b, lds, stream, a);
  }
  KVP_LAUNCH_CHECK();
  const dim3 cgrid(cdiv(kv->num_pairs * (a.g + a.fstep), 4));
  if (a.D == 64) hipLaunchKernelGGL((decode_attn_merge_kernel<64>), cgrid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((decode_attn_merge_kernel<128>), cgrid, dim3(256), 0, stream, a);
  KVP_LAUNCH_CHECK();
  return KVP_OK;
}

kvp_status kvp_launch_decode_attn(const void* q, int B, int Hq, const kvp_paged_kv* kv,
                                  const kvp_ring* ring, float sm_scale, float* out, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  (void)ws_bytes;
  return launch_attn(q, B, Hq, kv, ring, sm_scale, out, ws, stream, nullptr);
}

// The fused decode step: the delayed step's arguments (scores from s_in, or from the
// scorer: x_new for a linear one; for an MLP, x_new's split-K first-layer slices, which
// the stream kernel writes to part) and the attention, in the stream kernel plus the
// merge kernel.
kvp_status kvp_launch_decode_step(const kvp_scorer* sc, const void* x_new, float* part,
                                  const kvp_paged_kv* kv, const kvp_ring* ring, const void* k_new,
                                  const void* v_new, const float* s_in, int64_t ld_s, float* s_out,
                                  const float* tau, int* pos, const void* q, int B, int Hq,
                                  float sm_scale, float* out, void* ws, hipStream_t stream) {
  const StepArgs st = make_step_args(kv, ring, k_new, v_new, s_in, ld_s, 0.0f, tau, 0, pos, sc, x_new,
                                     s_out, part);
  if (sc && sc->kind == KVP_SCORER_MLP) {
    const SmallGemm gm = small_gemm_of(sc, x_new, st.ntok, sc->inner, part);
    return launch_attn(q, B, Hq, kv, ring, sm_scale, out, ws, stream, &st, &gm);
  }
  return launch_attn(q, B, Hq, kv, ring, sm_scale, out, ws, stream, &st);
}

