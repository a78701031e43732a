// GQA decode attention over the kept entries of the paged cache (gfx950).
//
// Method: KVzap digest (max5.ai), key points -- pruning shortens the sequence axis,
// which GQA alone does not; the attention reads only the kept entries.  BeaconKV
// briefing (jiinsi.com), body -- beacon entries at full precision and the others at
// low precision are read in one attention.
//
// One kernel per call, split-K with a deterministic in-kernel merge:
//   Every pair (b, h_kv) contributes a "region A" of virtual pages (its pool pages, then
//   its ring pages, padded to an even count) and, when a low-precision pool exists, a
//   "region B" (its int8 or int4 pages, padded to even).  The A regions are concatenated
//   into one page sequence and the B regions into another.  Each sequence is cut into
//   units: one large static unit per wave (most of the pages), then small dynamic units
//   that waves take from a ticket counter as they run out of work, so the waves of a
//   faster XCD absorb the tail of a slower one.  Unit boundaries depend only on the page
//   counts, never on timing, so every (unit, region) intersection -- a segment -- always
//   covers the same pages.  A wave walks its segments 32 tokens (two pages) at a time and
//   writes one partial (max, sum, output) record per segment; the wave that writes a
//   pair's last record (per-pair arrival counter) merges the pair's records in page order
//   and writes the output.  The result is therefore bit-identical from run to run.
//   Records are published across XCDs without cache maintenance: they are stored with
//   device-scope (sc1) stores, the writer waits for their completion before it bumps the
//   arrival counter, and the merging wave reads them with device-scope loads.
//   Record slot of the segment (region s, unit u) = base + s + u: along a sequence,
//   consecutive segments advance s or u (or both), so the slot is unique, and a region's
//   records occupy consecutive slots.
//
// Per 32-token step (bf16, head dim D, g query heads of one KV head):
//   S^T[32 tok x 16 heads] = K . Q^T on 16x16x32 bf16 MFMA (exact products, fp32
//   accumulation).  The K rows given to the two 16-row MFMA tiles are interleaved
//   so that each lane ends up holding the scores of 8 consecutive tokens of one head,
//   which is exactly the B-operand layout of the P.V MFMA that follows.
//   O^T[D x 16 heads] += V^T . P^T on MFMA, with P split into bf16 hi + lo parts so
//   the probabilities keep ~16 significant bits (V is exact in bf16).
//   V pages are stored dim-major ([d][16]) so V^T fragments are plain 16-byte loads.
// The bf16 stream keeps one step of K/V loads in flight and, one segment ahead, the next
// segment's query, length and block-table entries, so crossing from one pair to the
// next costs no memory round trip.
#include "kvp_internal.h"

namespace kvp {

constexpr int ATTN_WG_WAVES = 4;
constexpr int ATTN_GRID = 256;  // one work-group (4 waves) per CU on a 256-CU part
// int4 pools run two work-groups per CU (two waves per SIMD): a 32-token step of int4
// codes moves a quarter of a bf16 step's bytes but costs more instructions (nibble
// decode, the offset terms), and one wave per SIMD leaves its MFMA/VALU latencies
// exposed (measured on the BeaconKV int4 cache: 194 -> 171 us).  Every other cache keeps
// one wave per SIMD (the bf16 and int8 streams ran 1-4% slower with two).
constexpr int ATTN_MAX_WPE = 2;
constexpr int ATTN_MAX_NWAVES = ATTN_MAX_WPE * ATTN_GRID * ATTN_WG_WAVES;
// Register sets of code-pool loads in flight per wave (two 32-token steps): more sets
// (4 or 6) made the int4 stream 5-15% slower, fewer leave the loads exposed.
constexpr int ATTN_LP_SETS = 2;
static_assert(ATTN_GRID % 8 == 0, "units are numbered per XCD (8 XCDs)");

// Workspace: control words, per-pair arrival counts, then the records.  The counts and
// control words must be zero before the first call; every call leaves them zero.
constexpr int CTL_TICKET_A = 0, CTL_TICKET_B = 1, CTL_DONE = 2;
constexpr size_t ATTN_CTL_BYTES = 256;

// Dynamic units: about 1/20 of a wave's fair share each (2..8 pages), covering up to 12%
// of a sequence and at most two units per wave.
constexpr int ATTN_DYN_DIV = 20;
constexpr int ATTN_DYN_MAX_PAGES = 8;
constexpr int ATTN_DYN_PCT = 12;
constexpr int ATTN_DYN_PER_WAVE = 2;

struct AttnArgs {
  const void* q;
  float* out;
  int B, Hkv, Hq, g, D;
  kvp_paged_kv kv;
  kvp_ring ring;
  int has_ring;
  float scale_log2;  // sm_scale * log2(e)
  int* ctl;          // control words (tickets, done count)
  int* cnt;          // [num_pairs] record arrivals
  int* link;         // [num_pairs] next pair of a wave's list of pairs to merge
  float* part;       // records, rec_floats each
  int part_bytes;    // size of the record area (buffer-resource range)
  int rec_floats;    // g * (D + 2) rounded up to 4: o[g][D], then m[g], then l[g]
};

// -------------------------------------------------------------------------------
// Plan: page prefix P[] over the regions, computed by wave 0 of every work-group into
// LDS (one load per region, one wave scan, no barrier inside).
// -------------------------------------------------------------------------------
__device__ __forceinline__ int plan_regions(const AttnArgs& a) {
  return (a.kv.num_pages8 > 0 ? 2 : 1) * a.kv.num_pairs;
}

__device__ __forceinline__ int region_pages_of(int len, int extra) { return (cdiv(len, PAGE) + extra + 1) & ~1; }

// Wave 0: P[0] = 0, P[s + 1] = P[s] + pages of region s.  Each lane takes a run of
// regions; lengths are requested eight at a time so the loads overlap.
// The A regions' pool lengths go to Lens[] on the way.
__device__ __forceinline__ void compute_plan(const AttnArgs& a, int* P, int* Lens, int nseg) {
  const int lane = threadIdx.x & 63;
  const int np = a.kv.num_pairs;
  const int nring = a.has_ring ? a.ring.window / PAGE : 0;
  const int per = cdiv(nseg, 64);
  const int s0 = min(nseg, lane * per), s1 = min(nseg, s0 + per);
  int sum = 0;
  for (int b = s0; b < s1; b += 8) {
    int v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = b + i;
      v[i] = 0;
      if (s < s1) v[i] = (s < np) ? a.kv.length[s] : a.kv.length8[s - np];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = b + i;
      if (s < s1) {
        if (s < np) Lens[s] = v[i];
        const int n = region_pages_of(v[i], s < np ? nring : 0);
        P[s + 1] = n;
        sum += n;
      }
    }
  }
  int run = wave_incl_scan(sum) - sum;
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
  if (lane == 0) P[0] = 0;
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

// One page sequence (A: bf16/fp32 regions; B: low-precision regions) cut into units.
struct SeqSplit {
  int N;      // pages
  int s0;     // static unit size (0: no static band)
  int s1;     // dynamic unit size
  int ud;     // dynamic units
  int base;   // first record slot of the sequence
  int r0;     // first region of the sequence in P
  int pbase;  // P[r0]
};

__device__ __forceinline__ SeqSplit make_split(int N, int nw, int base, int r0, int pbase) {
  SeqSplit q;
  q.N = N;
  q.base = base;
  q.r0 = r0;
  q.pbase = pbase;
  q.s1 = 2;
  q.ud = 0;
  q.s0 = N > 0 ? ((cdiv(N, nw) + 1) & ~1) : 0;  // even; the last units may be short or empty
  return q;
}

// Units of a sequence: u < nw static ([u s0, (u + 1) s0)), then dynamic.
__device__ __forceinline__ int unit_of(const SeqSplit& q, int nw, int x) {
  const int st = nw * q.s0;
  return x < st ? x / max(1, q.s0) : nw + (x - st) / q.s1;
}

// Records (segments) of region s of the sequence, and the first one's unit.
__device__ __forceinline__ int region_records(const SeqSplit& q, int nw, const int* P, int s, int& uf) {
  const int p0 = P[s] - q.pbase, p1 = P[s + 1] - q.pbase;
  if (p1 <= p0) {
    uf = 0;
    return 0;
  }
  uf = unit_of(q, nw, p0);
  return unit_of(q, nw, p1 - 1) - uf + 1;
}

// -------------------------------------------------------------------------------
// Units and segments
// -------------------------------------------------------------------------------
struct SegDesc {
  int s;         // region index in P
  int vlo, vhi;  // pages of the region covered by the segment
  int u;         // unit
  int rev;       // walk backwards
  int ok;        // 0: no more work
};

// Walks a wave's units of one sequence: its static unit, then dynamic units by ticket.
// The ticket of the next unit is requested when a unit starts, so its latency hides
// behind that unit's pages.
struct UnitIter {
  SeqSplit sp;
  int nw, gw, nreg;
  int* ticket;
  int started, have;
  int u, X0, X1, rev;  // current unit, its pages in P coordinates
  int r, r_end;        // next region to emit, last region (walk order)
  int tk_v;            // lane 0: the requested ticket
  int tk_pending;
  int finished;        // a ticket past the end was drawn: no further requests
};

__device__ __forceinline__ void iter_init(UnitIter& it, const SeqSplit& sp, int nw, int gw, int nreg, int* ticket) {
  it.sp = sp;
  it.nw = nw;
  it.gw = gw;
  it.nreg = nreg;
  it.ticket = ticket;
  it.started = 0;
  it.have = 0;
  it.tk_v = 0;
  it.tk_pending = 0;
  it.finished = 0;
}

__device__ __forceinline__ int request_ticket(int* ticket) {
  int v = 0;
  if ((threadIdx.x & 63) == 0) v = atomicAdd(ticket, 1);
  return v;
}

__device__ __forceinline__ bool iter_next_unit(UnitIter& it, const int* P) {
  if (it.finished) return false;
  int u = -1;
  if (!it.started) {
    it.started = 1;
    if (it.sp.s0 > 0 && it.gw * it.sp.s0 < it.sp.N) u = it.gw;  // the last static units may be empty
  }
  if (u < 0) {
    if (it.sp.ud == 0) {
      it.finished = 1;
      return false;
    }
    const int t = __builtin_amdgcn_readfirstlane(it.tk_pending ? it.tk_v : request_ticket(it.ticket));
    it.tk_pending = 0;
    if ((unsigned)t >= (unsigned)it.sp.ud) {
      it.finished = 1;
      return false;
    }
    u = it.nw + t;
  }
  if (it.sp.ud > 0) {
    it.tk_v = request_ticket(it.ticket);
    it.tk_pending = 1;
  }
  int x0, x1;
  if (u < it.nw) {
    x0 = u * it.sp.s0;
    x1 = min(it.sp.N, x0 + it.sp.s0);
    it.rev = u & 1;  // odd static units walk backwards: opposite directions keep the
                     // 1024 streams from settling on the same HBM channels (measured: 10%
                     // at one keep ratio); the order only changes rounding inside a record
  } else {
    x0 = it.nw * it.sp.s0 + (u - it.nw) * it.sp.s1;
    x1 = min(it.sp.N, x0 + it.sp.s1);
    it.rev = 0;
  }
  it.u = u;
  it.X0 = it.sp.pbase + x0;
  it.X1 = it.sp.pbase + x1;
  const int rf = seg_search(P, it.sp.r0, it.sp.r0 + it.nreg, it.X0);
  const int rl = seg_search(P, it.sp.r0, it.sp.r0 + it.nreg, it.X1 - 1);
  it.r = it.rev ? rl : rf;
  it.r_end = it.rev ? rf : rl;
  it.have = 1;
  return true;
}

__device__ __forceinline__ SegDesc iter_next_seg(UnitIter& it, const int* P) {
  SegDesc d;
  d.ok = 0;
  for (;;) {
    if (!it.have && !iter_next_unit(it, P)) return d;
    while (it.have) {
      const int r = it.r;
      if (r == it.r_end) it.have = 0;
      else it.r += it.rev ? -1 : 1;
      const int p0 = __builtin_amdgcn_readfirstlane(P[r]), p1 = __builtin_amdgcn_readfirstlane(P[r + 1]);
      if (p1 > p0) {
        d.s = r;
        d.vlo = max(it.X0, p0) - p0;
        d.vhi = min(it.X1, p1) - p0;
        d.u = it.u;
        d.rev = it.rev;
        d.ok = 1;
        return d;
      }
    }
  }
}

// -------------------------------------------------------------------------------
// Records: publication, arrival, merge
// -------------------------------------------------------------------------------
struct Splits {
  SeqSplit A, B;
  int nw, lp;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_rsrc(const AttnArgs& a) {
  return __builtin_amdgcn_make_buffer_rsrc(a.part, (short)0, a.part_bytes, 0x00020000);
}
constexpr int SC1 = 16;  // buffer cache policy: device scope (coherent across XCDs)

__device__ __forceinline__ void rec_store4(__amdgpu_buffer_rsrc_t r, int off_f, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off_f * 4, 0, SC1);
}
__device__ __forceinline__ void rec_store1(__amdgpu_buffer_rsrc_t r, int off_f, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off_f * 4, 0, SC1);
}
__device__ __forceinline__ float rec_load1(__amdgpu_buffer_rsrc_t r, int off_f) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off_f * 4, 0, SC1));
}

// Records of a pair: A-sequence slots [slA, slA + nA), then B-sequence slots.
struct PairRecs {
  int slA, nA, slB, nB;
};

__device__ __forceinline__ PairRecs pair_records(const Splits& sp, const int* P, int np, int pair) {
  PairRecs pr;
  int uf = 0;
  pr.nA = region_records(sp.A, sp.nw, P, pair, uf);
  pr.slA = sp.A.base + pair + uf;
  pr.nB = 0;
  pr.slB = 0;
  if (sp.lp) {
    pr.nB = region_records(sp.B, sp.nw, P, np + pair, uf);
    pr.slB = sp.B.base + pair + uf;
  }
  return pr;
}

__device__ __forceinline__ int slot_of(const Splits& sp, const SegDesc& d, int np) {
  return d.s < np ? sp.A.base + d.s + d.u : sp.B.base + (d.s - np) + d.u;
}

__device__ __forceinline__ f32x4 rec_load4(__amdgpu_buffer_rsrc_t r, int off_f) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off_f * 4, 0, SC1));
}

// Merge of a pair's records in slot order by one wave, 64 records per round (online
// rescale between rounds).  Lane r holds record r's per-head max and sum; the outputs
// o[g][D] are read as 16-byte pieces, lane l owning pieces c = l + 64 i (head 4 c / D),
// RB records per batch with all their loads in flight; the first batch is requested
// together with the maxima and sums.
template <int D, int EC>  // EC: pieces per lane per record, ceil(g D / 256)
__device__ __forceinline__ void merge_pair(const AttnArgs& a, const PairRecs& pr, int pair) {
  constexpr int RB = EC >= 16 ? 1 : 16 / EC;
  constexpr int PPH = D / 4;         // pieces per head
  constexpr int LPH = 64 / PPH;      // heads covered by one row of 64 pieces
  const int lane = threadIdx.x & 63, g = a.g, rf = a.rec_floats;
  const int n = pr.nA + pr.nB;
  const int npc = g * PPH;
  const __amdgpu_buffer_rsrc_t rs = rec_rsrc(a);
  auto slot = [&](int k) { return k < pr.nA ? pr.slA + k : pr.slB + (k - pr.nA); };
  float M[16], den[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    M[h] = neg_inf();
    den[h] = 0.f;
  }
  f32x4 acc[EC];
#pragma unroll
  for (int i = 0; i < EC; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < n; r0 += 64) {
    const int nr = min(64, n - r0);
    // maxima and sums of this round's records (lane = record), and the first batch
    const int mb = slot(r0 + min(lane, nr - 1)) * rf + g * D;
    float mv[16], lv[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      mv[h] = neg_inf();
      lv[h] = 0.f;
      if (h < g) {
        mv[h] = rec_load1(rs, mb + h);
        lv[h] = rec_load1(rs, mb + g + h);
      }
    }
    f32x4 o[RB][EC];
    auto issue = [&](int k0) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int b = slot(r0 + min(k0 + r, nr - 1)) * rf;
#pragma unroll
        for (int i = 0; i < EC; ++i) {
          const int c = lane + 64 * i;
          o[r][i] = (c < npc) ? rec_load4(rs, b + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    };
    issue(0);
    float w[16], sc[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      w[h] = 0.f;
      sc[h] = 1.f;
      if (h < g) {
        const float mh = (lane < nr) ? mv[h] : neg_inf();
        const float Mn = fmaxf(M[h], wave_max(mh));
        sc[h] = (Mn == neg_inf()) ? 1.f : exp2f(M[h] - Mn);
        w[h] = (mh == neg_inf()) ? 0.f : exp2f(mh - Mn);
        den[h] = den[h] * sc[h] + wave_sum(w[h] * lv[h]);
        M[h] = Mn;
      }
    }
    // earlier rounds' sums move to the new maxima
#pragma unroll
    for (int i = 0; i < EC; ++i) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < LPH; ++q)
        if (lane / PPH == q) s = sc[LPH * i + q < 16 ? LPH * i + q : 15];
      acc[i] *= s;
    }
    for (int k0 = 0; k0 < nr; k0 += RB) {
      if (k0 > 0) issue(k0);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        if (k0 + r < nr) {
#pragma unroll
          for (int i = 0; i < EC; ++i) {
            float wl = 0.f;
#pragma unroll
            for (int q = 0; q < LPH; ++q) {
              const int h = LPH * i + q < 16 ? LPH * i + q : 15;
              const float wh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w[h]), k0 + r));
              if (lane / PPH == q) wl = wh;
            }
            acc[i] += wl * o[r][i];
          }
        }
      }
    }
  }
  const int b = pair / a.Hkv, hk = pair % a.Hkv;
  float* out = a.out + ((int64_t)b * a.Hq + (int64_t)hk * g) * D;
#pragma unroll
  for (int i = 0; i < EC; ++i) {
    const int c = lane + 64 * i;
    if (c < npc) {
      float dn = 0.f;
#pragma unroll
      for (int q = 0; q < LPH; ++q)
        if (lane / PPH == q) dn = den[LPH * i + q < 16 ? LPH * i + q : 15];
      const float inv = dn > 0.f ? 1.0f / dn : 0.f;
      *reinterpret_cast<f32x4*>(out + 4 * c) = acc[i] * inv;
    }
  }
}

template <int D>
__device__ __forceinline__ void merge_dispatch(const AttnArgs& a, const PairRecs& pr, int pair) {
  const int npc = a.g * D / 4;
  if (npc <= 64) merge_pair<D, 1>(a, pr, pair);
  else if (npc <= 128) merge_pair<D, 2>(a, pr, pair);
  else if (npc <= 256) merge_pair<D, 4>(a, pr, pair);
  else merge_pair<D, 8>(a, pr, pair);
}

// A published record waiting for its arrival (pend), an arrival whose count has not
// been looked at yet (iss), and the pairs this wave has won and still has to merge: a
// list threaded through the per-pair link array of the workspace (each pair is won by
// exactly one wave per call), merged once the wave's stream is over so the merge's
// registers never compete with the stream's.
struct Arrivals {
  int pend, pend_pair;
  int iss, iss_pair, iss_old;
  int won;  // first pair of the list, -1 when empty
};

__device__ __forceinline__ void arrivals_init(Arrivals& ar) {
  ar.pend = 0;
  ar.iss = 0;
  ar.won = -1;
}

// The record stores must be complete (device scope) before the count moves: wait for
// every outstanding vector memory operation, then bump the pair's count.
__device__ __forceinline__ void arrival_issue(const AttnArgs& a, Arrivals& ar) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int v = 0;
  if ((threadIdx.x & 63) == 0) v = atomicAdd(a.cnt + ar.pend_pair, 1);
  ar.iss = 1;
  ar.iss_pair = ar.pend_pair;
  ar.iss_old = v;
  ar.pend = 0;
}

// The wave that brings a pair's count to its record total clears the count for the next
// call and puts the pair on its list (merged later, see Arrivals).  A count beyond the
// total can only come from a workspace that was not zeroed before its first use:
// flagged in kv.err.
template <int D>
__device__ __forceinline__ void arrival_check(const AttnArgs& a, const Splits& sp, const int* P, Arrivals& ar) {
  const int old = __builtin_amdgcn_readfirstlane(ar.iss_old);
  ar.iss = 0;
  const PairRecs pr = pair_records(sp, P, a.kv.num_pairs, ar.iss_pair);
  const int n = pr.nA + pr.nB;
  if (old == n - 1) {
    if ((threadIdx.x & 63) == 0) {
      __hip_atomic_store(a.cnt + ar.iss_pair, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.link[ar.iss_pair] = ar.won;
    }
    ar.won = ar.iss_pair;
  } else if ((unsigned)old >= (unsigned)n) {
    if ((threadIdx.x & 63) == 0) atomicOr(a.kv.err, KVP_ERR_ATTN_WS);
  }
}

template <int D>
__device__ __forceinline__ void merge_won(const AttnArgs& a, const Splits& sp, const int* P, Arrivals& ar) {
  int pair = ar.won;
  while (pair >= 0) {
    const int next = __builtin_amdgcn_readfirstlane(a.link[pair]);
    merge_dispatch<D>(a, pair_records(sp, P, a.kv.num_pairs, pair), pair);
    pair = next;
  }
  ar.won = -1;
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
  int kind;           // 0 main, 1 ring, 2 padding
  int nvalid;         // main: valid slots; ring: ring page index
};

// Page v of region A of `pair` (walk position w, for the block-table chunk in bt).
template <int D>
__device__ __forceinline__ PageRef region_a_page(const AttnArgs& a, int pair, int v, int w, int bt, int npm,
                                                 int len, int nring) {
  PageRef r;
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
  } else {
    r.k = nullptr;
    r.v = nullptr;
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
                                           int nring, PageRef& X, PageRef& Y) {
  const int vX = d.rev ? d.vhi - 2 - 2 * k : d.vlo + 2 * k;
  const int wX = d.rev ? 2 * k + 1 : 2 * k, wY = d.rev ? 2 * k : 2 * k + 1;
  X = region_a_page<D>(a, d.s, vX, wX, bt, npm, len, nring);
  Y = region_a_page<D>(a, d.s, vX + 1, wY, bt, npm, len, nring);
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
    return b;
  }
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
  const uint16_t* rowA = kbase + (tA & 15) * D + (D / 4) * j;
  const uint16_t* rowB = kbase + (tB & 15) * D + (D / 4) * j;
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
  const uint16_t* vcol = vbase + m * PAGE + 8 * (j & 1);
#pragma unroll
  for (int t = 0; t < D / 16; ++t) f.v[t] = *reinterpret_cast<const u32x4*>(vcol + t * 16 * PAGE);
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

template <int D>
__device__ __forceinline__ void pv_step(const Bf16Frags<D>& f, SoftmaxState<D>& st, bf16x8 phi,
                                        bf16x8 plo, uint32_t vbits, bool all_valid) {
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

// End of a segment of pair `pair` whose state is in the MFMA layout (lane: head n =
// lane % 16, dims 16 t + 4 (lane / 16) + 0..3): a pair with a single record is finished
// here; otherwise the record is published and its arrival left pending.
template <int D>
__device__ __forceinline__ void segment_done(const AttnArgs& a, const Splits& sp, const int* P, int pair, int slot,
                             SoftmaxState<D>& st, Arrivals& ar) {
  const int lane = threadIdx.x & 63, n = lane & 15, j = lane >> 4;
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const PairRecs pr = pair_records(sp, P, a.kv.num_pairs, pair);
  if (pr.nA + pr.nB == 1) {
    const int b = pair / a.Hkv, h = pair % a.Hkv;
    float* out = a.out + ((int64_t)b * a.Hq + h * a.g + n) * D;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    if (n < a.g) {
#pragma unroll
      for (int t = 0; t < D / 16; ++t) *reinterpret_cast<f32x4*>(out + 16 * t + 4 * j) = st.o[t] * inv;
    }
    return;
  }
  const __amdgpu_buffer_rsrc_t rs = rec_rsrc(a);
  const int base = slot * a.rec_floats;
  if (n < a.g) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) rec_store4(rs, base + n * D + 16 * t + 4 * j, st.o[t]);
    if (j == 0) {
      rec_store1(rs, base + a.g * D + n, st.m);
      rec_store1(rs, base + a.g * D + a.g + n, l);
    }
  }
  ar.pend = 1;
  ar.pend_pair = pair;
}

// -------------------------------------------------------------------------------
// The bf16 stream over region-A segments.  One step of K/V loads is in flight behind
// the math; the segment after the next one is looked up (block-table entries requested)
// one iteration after a switch, so every segment's first pages are addressable by the
// time the previous segment's last step issues their loads; the next pair's queries are
// loaded together with its first K.  Record arrivals are issued right after the next
// step's QK MFMAs, when only that step's V loads are outstanding, so waiting for the
// record stores costs no stream stall.
// -------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void stream_a_bf16(const AttnArgs& a, const Splits& sp, const int* P, const int* Lens,
                                              UnitIter& it, Arrivals& ar) {
  const int lane = threadIdx.x & 63, j = lane >> 4;
  const int np = a.kv.num_pairs;
  const int nring = a.has_ring ? a.ring.window / PAGE : 0;
  SegDesc cur = iter_next_seg(it, P);
  if (!cur.ok) return;
  SegDesc nxt = iter_next_seg(it, P);
  SegDesc nx2;
  nx2.ok = 0;
  int bt_cur0 = load_bt_chunk(a, cur, 0), bt_cur1 = 0;
  int bt_nxt = nxt.ok ? load_bt_chunk(a, nxt, 0) : 0;
  int bt_nx2 = 0;
  bool fetch_nx2 = nxt.ok;
  int len = __builtin_amdgcn_readfirstlane(Lens[cur.s]);
  int npm = cdiv(len, PAGE);
  int nst = (cur.vhi - cur.vlo) >> 1;
  bool chunk_load = nst > 32;  // chunk 1 of the current segment still to request
  int cc = 0;                  // block-table chunk of the current step
  bf16x8 qf[D / 32], qn[D / 32];
  load_q<D>(a, cur.s, qf);
  PageRef x, y;
  step_pages<D>(a, cur, 0, bt_cur0, npm, len, nring, x, y);
  Bf16Frags<D> f;
  load_k<D>(a, f, cur.s, x, y, lane);
  load_v<D>(f, x, y, lane);
  SoftmaxState<D> st;
  state_reset(st);
  int k = 0;
  for (;;) {
    const bool lastk = (k + 1 == nst);
    const bool have_next = !lastk || nxt.ok;
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
      step_pages<D>(a, cur, k + 1, (cc & 1) ? bt_cur1 : bt_cur0, npm, len, nring, xn, yn);
    } else if (nxt.ok) {
      const int lenn = __builtin_amdgcn_readfirstlane(Lens[nxt.s]);
      step_pages<D>(a, nxt, 0, bt_nxt, cdiv(lenn, PAGE), lenn, nring, xn, yn);
      pair_n = nxt.s;
      load_q<D>(a, nxt.s, qn);
    }
    const uint32_t vb = lane_valid_bits(f.rp0, f.rp1, x, y, j);
    const bool allv = __ballot(vb != 0xffu) == 0;
    f32x4 sA, sB;
    qk_step<D>(f, qf, sA, sB);
    if (ar.pend) arrival_issue(a, ar);
    load_k<D>(a, f, pair_n, xn, yn, lane);
    bf16x8 phi, plo;
    if (softmax_step<D>(a, sA, sB, st, vb, allv, phi, plo)) pv_step<D>(f, st, phi, plo, vb, allv);
    load_v<D>(f, xn, yn, lane);
    if (lastk) {
      segment_done<D>(a, sp, P, cur.s, sp.A.base + cur.s + cur.u, st, ar);
      state_reset(st);
    }
    if (ar.iss) arrival_check<D>(a, sp, P, ar);
    // look-ahead requests (rare)
    if (chunk_load) {
      bt_cur1 = load_bt_chunk(a, cur, 1);
      chunk_load = false;
    }
    if (fetch_nx2) {
      nx2 = iter_next_seg(it, P);
      if (nx2.ok) bt_nx2 = load_bt_chunk(a, nx2, 0);
      fetch_nx2 = false;
    }
    if (!have_next) break;
    x = xn;
    y = yn;
    if (lastk) {
      cur = nxt;
      nxt = nx2;
      bt_cur0 = bt_nxt;
      bt_nxt = bt_nx2;
      len = __builtin_amdgcn_readfirstlane(Lens[cur.s]);
      npm = cdiv(len, PAGE);
      nst = (cur.vhi - cur.vlo) >> 1;
      chunk_load = nst > 32;
      cc = 0;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qf[kk] = qn[kk];
      fetch_nx2 = nxt.ok;
      nx2.ok = 0;
      k = 0;
    } else {
      ++k;
    }
  }
  if (ar.pend) arrival_issue(a, ar);
  if (ar.iss) arrival_check<D>(a, sp, P, ar);
  (void)np;
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

// 8 codes of a fragment: two dwords of int8 codes or one dword of int4 codes.
template <int BITS> struct LpWord { typedef u32x2 T; };
template <> struct LpWord<4> { typedef uint32_t T; };
__device__ __forceinline__ u32x4 lp_to_bf16x8(u32x2 w) { return i8x8_to_bf16x8(w[0], w[1]); }
__device__ __forceinline__ u32x4 lp_to_bf16x8(uint32_t w) { return i4x8_to_bf16x8(w); }

template <int D, int BITS>
struct LpFrags {
  typedef typename LpWord<BITS>::T W;
  W kA[D / 32];  // 8 K codes per MFMA K-step, score tile A row
  W kB[D / 32];
  W v[D / 16];   // 8 V^T codes per output tile
  f32x4 ks[2];   // K scales of this lane's 8 tokens
  f32x4 vs[2];   // V scales of this lane's 8 tokens
};

// Byte offsets scale with the code width: a K row is D * BITS / 8 bytes, a V^T row
// 16 * BITS / 8.
template <int D, int BITS>
__device__ __forceinline__ void load_lp_k(const AttnArgs& a, LpFrags<D, BITS>& f, int pgX, int pgY, int lane) {
  typedef typename LpWord<BITS>::T W;
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

template <int D, int BITS>
__device__ __forceinline__ void load_lp_v(const AttnArgs& a, LpFrags<D, BITS>& f, int pgX, int pgY, int lane) {
  typedef typename LpWord<BITS>::T W;
  const int m = lane & 15, j = lane >> 4;
  const int pgT = (j < 2) ? pgX : pgY;
  const int8_t* vcol = a.kv.v8_pages + ((int64_t)pgT * PAGE * D + m * PAGE + 8 * (j & 1)) * BITS / 8;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) f.v[t] = *reinterpret_cast<const W*>(vcol + t * 16 * PAGE * BITS / 8);
  const float* vsc = a.kv.v8_scale + (int64_t)pgT * PAGE + 8 * (j & 1);
  f.vs[0] = *reinterpret_cast<const f32x4*>(vsc);
  f.vs[1] = *reinterpret_cast<const f32x4*>(vsc + 4);
}

template <int D, int BITS, int NSET>
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
    auto qk = [&](const LpFrags<D, BITS>& f, float (&s)[8], float (&vsc)[8]) {
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
    auto pv = [&](const LpFrags<D, BITS>& f, const float (&p)[8], const float (&vsc)[8]) {
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
    LpFrags<D, BITS> f[NSET];
#pragma unroll
    for (int r = 0; r < NSET; ++r) {
      load_lp_k<D, BITS>(a, f[r], page(vat(r)), page(vat(r) + 1), lane);
      load_lp_v<D, BITS>(a, f[r], page(vat(r)), page(vat(r) + 1), lane);
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
        load_lp_k<D, BITS>(a, f[r], page(vna), page(vna + 1), lane);
        load_lp_k<D, BITS>(a, f[r + 1], page(vnb), page(vnb + 1), lane);
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
        load_lp_v<D, BITS>(a, f[r], page(vna), page(vna + 1), lane);
        load_lp_v<D, BITS>(a, f[r + 1], page(vnb), page(vnb + 1), lane);
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
__device__ __forceinline__ void run_region_a_f32(const AttnArgs& a, const Splits& sp, const int* P, int pair, int v0, int v1,
                                 int slot, float* wlds, Arrivals& ar) {
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
  // end of the segment: finish a single-record pair here, else publish the record
  const PairRecs pr = pair_records(sp, P, a.kv.num_pairs, pair);
  if (pr.nA + pr.nB == 1) {
    float* out = a.out + ((int64_t)b * a.Hq + h * g) * D;
    for (int n = 0; n < g; ++n) {
      const float inv = lrun[n] > 0.f ? 1.0f / lrun[n] : 0.f;
      for (int e = 0; e < D / 64; ++e) out[n * D + lane + 64 * e] = o[n][e] * inv;
    }
    return;
  }
  const __amdgpu_buffer_rsrc_t rs = rec_rsrc(a);
  const int base = slot * a.rec_floats;
  for (int n = 0; n < g; ++n) {
    for (int e = 0; e < D / 64; ++e) rec_store1(rs, base + n * D + lane + 64 * e, o[n][e]);
    if (lane == 0) {
      rec_store1(rs, base + g * D + n, mrun[n]);
      rec_store1(rs, base + g * D + g + n, lrun[n]);
    }
  }
  ar.pend = 1;
  ar.pend_pair = pair;
}

// Region-B (low-precision) and fp32 segments: one segment at a time (its query, length
// and block table fetched at its start), arrivals issued at its end.
template <int D, bool F32, int BITS>
__device__ __forceinline__ void stream_segments(const AttnArgs& a, const Splits& sp, const int* P, UnitIter& it,
                                                float* wlds, Arrivals& ar) {
  const int np = a.kv.num_pairs;
  for (;;) {
    const SegDesc d = iter_next_seg(it, P);
    if (!d.ok) break;
    if constexpr (F32) {
      run_region_a_f32<D>(a, sp, P, d.s, d.vlo, d.vhi, slot_of(sp, d, np), wlds, ar);
    } else {
      SoftmaxState<D> st;
      run_region_b_lp<D, BITS, ATTN_LP_SETS>(a, d.s - np, d.vlo, d.vhi, d.rev != 0, st);
      segment_done<D>(a, sp, P, d.s - np, slot_of(sp, d, np), st, ar);
    }
    if (ar.pend) arrival_issue(a, ar);
    if (ar.iss) arrival_check<D>(a, sp, P, ar);
  }
}

// -------------------------------------------------------------------------------
// The kernel
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
  int* P = lds;
  int* Lens = lds + nseg + 1;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wid == 0) compute_plan(a, P, Lens, nseg);
  __syncthreads();
  const int nw = gridDim.x * ATTN_WG_WAVES;
  // Work-groups are dispatched round-robin over the 8 XCDs; numbering the static units so
  // that each XCD takes one contiguous eighth of the sequence evens out the XCDs' finish
  // times (measured: 1-3 us at the 361 MB and 543 MB caches).
  const int gw = ((blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8) * ATTN_WG_WAVES + wid;
  Splits sp;
  sp.nw = nw;
  sp.lp = LP ? 1 : 0;
  const int NA = __builtin_amdgcn_readfirstlane(P[np]);
  sp.A = make_split(NA, nw, 0, 0, 0);
  sp.B = make_split(LP ? __builtin_amdgcn_readfirstlane(P[nseg]) - NA : 0, nw, np + nw + sp.A.ud, np, NA);
  // pairs with nothing visible: zeros
  for (int p = gw; p < np; p += nw) {
    const PairRecs pr = pair_records(sp, P, np, p);
    if (pr.nA + pr.nB == 0) {
      const int b = p / a.Hkv, hk = p % a.Hkv;
      float* out = a.out + ((int64_t)b * a.Hq + (int64_t)hk * a.g) * a.D;
      for (int e = threadIdx.x & 63; e < a.g * a.D; e += 64) out[e] = 0.f;
    }
  }
  Arrivals ar;
  arrivals_init(ar);
  float* wlds = nullptr;
  if constexpr (F32) wlds = reinterpret_cast<float*>(lds + 2 * nseg + 2) + wid * (16 * D + 16 * 32);
  UnitIter it;
  iter_init(it, sp.A, nw, gw, np, a.ctl + CTL_TICKET_A);
  if constexpr (F32) {
    stream_segments<D, true, 8>(a, sp, P, it, wlds, ar);
  } else {
    stream_a_bf16<D>(a, sp, P, Lens, it, ar);
    if constexpr (LP) {
      iter_init(it, sp.B, nw, gw, np, a.ctl + CTL_TICKET_B);
      if (a.kv.lp_bits == 4) stream_segments<D, false, 4>(a, sp, P, it, nullptr, ar);
      else stream_segments<D, false, 8>(a, sp, P, it, nullptr, ar);
    }
  }
  merge_won<D>(a, sp, P, ar);
  // The last wave out clears the tickets for the next call.  Every wave takes exactly one
  // ticket past the end of each sequence it drew from, so the totals are known; other
  // values mean the control words were not zero at the start.
  int old = 0;
  if ((threadIdx.x & 63) == 0) old = atomicAdd(a.ctl + CTL_DONE, 1);
  old = __builtin_amdgcn_readfirstlane(old);
  if (old == nw - 1 && (threadIdx.x & 63) == 0) {
    const int ta = __hip_atomic_exchange(a.ctl + CTL_TICKET_A, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int tb = __hip_atomic_exchange(a.ctl + CTL_TICKET_B, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.ctl + CTL_DONE, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int ea = sp.A.ud > 0 ? sp.A.ud + nw : 0;
    const int eb = (LP && sp.B.ud > 0) ? sp.B.ud + nw : 0;
    if (ta != ea || tb != eb) atomicOr(a.kv.err, KVP_ERR_ATTN_WS);
  } else if ((unsigned)old >= (unsigned)nw && (threadIdx.x & 63) == 0) {
    atomicOr(a.kv.err, KVP_ERR_ATTN_WS);
  }
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

// Record slots of one sequence: regions + static units + dynamic units (at most 3 per
// wave plus one, see make_split), for the largest launch (two waves per SIMD).
static size_t attn_max_slots(int num_pairs) {
  return 2 * ((size_t)num_pairs + 4 * (size_t)ATTN_MAX_NWAVES + 1);
}

static size_t attn_rec_floats(int g, int D) { return ((size_t)g * (D + 2) + 3) & ~(size_t)3; }

static size_t attn_cnt_bytes(int num_pairs) { return (((size_t)num_pairs * sizeof(int)) + 255) & ~(size_t)255; }
// Workspace: [control words][arrival counts][pair links][records]; only the first two
// must start at zero.

extern "C" size_t kvp_decode_attn_workspace_size(int32_t B, int32_t Hq, int32_t num_pairs,
                                                 int32_t head_dim) {
  if (B <= 0 || Hq <= 0 || num_pairs <= 0 || head_dim <= 0 || num_pairs % B != 0) return 0;
  const int Hkv = num_pairs / B;
  if (Hq % Hkv != 0) return 0;
  const int g = Hq / Hkv;
  return ATTN_CTL_BYTES + 2 * attn_cnt_bytes(num_pairs) + attn_max_slots(num_pairs) * attn_rec_floats(g, head_dim) * sizeof(float);
}

kvp_status kvp_launch_decode_attn(const void* q, int B, int Hq, const kvp_paged_kv* kv,
                                  const kvp_ring* ring, float sm_scale, float* out, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  AttnArgs a;
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
  char* w = reinterpret_cast<char*>(ws);
  a.ctl = reinterpret_cast<int*>(w);
  a.cnt = reinterpret_cast<int*>(w + ATTN_CTL_BYTES);
  a.link = reinterpret_cast<int*>(w + ATTN_CTL_BYTES + attn_cnt_bytes(kv->num_pairs));
  a.part = reinterpret_cast<float*>(w + ATTN_CTL_BYTES + 2 * attn_cnt_bytes(kv->num_pairs));
  const size_t part_bytes = ws_bytes - ATTN_CTL_BYTES - 2 * attn_cnt_bytes(kv->num_pairs);
  if (part_bytes > 0x7fffffffu) return KVP_E_UNSUPPORTED;  // buffer offsets are 32-bit
  a.part_bytes = (int)part_bytes;
  a.rec_floats = (int)attn_rec_floats(a.g, a.D);
  const bool f32 = kv->dtype == KVP_F32;
  const bool lp = kv->num_pages8 > 0;
  const size_t lds = attn_lds_bytes(kv->num_pairs, a.D, f32, lp);
  if (lds > 160 * 1024) return KVP_E_UNSUPPORTED;
  const dim3 g1(ATTN_GRID), b(256);
  if (f32) {
    if (a.D == 64) hipLaunchKernelGGL((decode_attn_kernel<64, true, false, 1>), g1, b, lds, stream, a);
    else hipLaunchKernelGGL((decode_attn_kernel<128, true, false, 1>), g1, b, lds, stream, a);
  } else if (lp && kv->lp_bits == 4) {
    const dim3 g2(ATTN_GRID * 2);
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
  return KVP_OK;
}

size_t kvp_attn_lds_bytes_host(int num_pairs, int D, bool f32, bool lp) {
  return attn_lds_bytes(num_pairs, D, f32, lp);
}
