// Prefill attention under eviction (gfx950): every prompt position attends, causally,
// to the keys the cache still holds for it.
//
// Method: DMS briefing, "Delayed Eviction" (a flagged token stays readable for a window
// of steps, then leaves the cache); KVzap digest, key points (low-scoring entries are
// removed, the most recent ones always kept).  Prompt position i sees key j iff
// j <= i and (keep_j or i - j < W): what the decode step at length i + 1 sees.
//
// Work decomposition: one work-group (8 waves) per (pair (b, h_kv), block of
// PB = 256 / g positions).  Its 256 query rows are the g query heads of the pair times
// the PB positions; each wave owns 32 rows as two 16-row column tiles (one head, 16
// consecutive positions each).  The keys a block needs are
//   - the kept keys below lo64 = floor64(max(0, i0 - W + 1)): every row of the block
//     sees all of them, so they carry no mask except the last tile's tail; they are
//     gathered in ascending order through kept_idx, and
//   - the band [lo64, min(T, i0 + PB)): dense, masked per row with the keep bits.
// Both are walked in 64-key tiles staged through LDS: K row-major with its 16-byte
// chunks swizzled per row, V transposed to [d][key] on the way in (register byte
// permutes, then 8-byte LDS writes), so every MFMA operand is one 16-byte LDS read.
// Two register sets and two LDS buffers alternate (one barrier per tile): a tile's K/V
// rows are requested three tiles before their use and stored one tile before it; its
// kept_idx entries are read a tile earlier than the rows.  One 8-wave
// work-group per CU (two waves per SIMD): 256 rows share each staged tile, which halves
// the gathered bytes per flop against 4-wave groups (measured 9% faster).
//
// Per 32-key chunk and column tile: S^T = K Q^T on 16x16x32 bf16 MFMA (exact
// products, fp32 accumulation), with the K rows of the two 16-row MFMA tiles
// interleaved so each lane holds the scores of 8 consecutive keys of one query row --
// the B-operand layout of the P.V product that follows.  Online softmax in fp32 (log2
// domain); O^T += V^T P^T with P split into bf16 hi + lo parts (~16 significant bits),
// both column tiles' P first so that each V^T fragment is read from LDS once for both
// (LDS reads are what the kernel shares its time with the matrix pipe on).
// Work-groups are numbered heavy-first (the last position blocks see the most keys);
// the 32 blocks an XCD runs at a time are adjacent blocks of one pair, so the kept keys
// they all read come from that XCD's L2; an XCD finishes a pair before the next, and
// consecutive runs walk the kept keys in opposite directions, so a run starts on what
// the previous run left in L2.  Query rows (read once) are loaded and outputs (written
// once) stored non-temporally, so they do not evict the shared keys; outputs are staged
// through LDS first so that every store covers whole lines.  The pairs of an XCD mix KV
// heads (the kept fraction differs between heads).
#include "kvp_internal.h"

namespace kvp {

constexpr int PF_KT = 64;      // keys per LDS tile
constexpr int PF_THREADS = 512;
constexpr int PF_WAVES = PF_THREADS / 64;
constexpr int PF_ROWS = 32 * PF_WAVES;  // query rows per work-group
constexpr int PF_GS = 32;               // work-groups per run: one per CU of an XCD
// key slots of a tile each thread stages: 64 slots x D/8 chunks over the threads
__host__ __device__ constexpr int pf_kg(int D) { return 64 * (D / 8) / PF_THREADS; }
constexpr float PF_HEADROOM = 8.0f;  // log2 units a score may pass the reference by

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* out;
  const uint32_t* keep_bits;
  const int* kept_idx;
  int Hq, Hkv, T, g, pb, nblk, window, words, num_pairs;
  int nx, per_x;  // XCD groups (8, or 1 when num_pairs % 8 != 0) and pairs per group
  float scale_log2;  // sm_scale * log2(e)
};

// K tile: row r (key slot), 16-byte chunk c stored at chunk c ^ k_swz(r).  The 16 rows
// one MFMA operand read touches (slots 8q + m and 8q + 4 + m, q, m < 4) map to 16
// distinct chunk positions (D = 128) or to distinct (row parity, chunk) pairs (D = 64).
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (D == 128) return (((r >> 3) & 3) << 2) | (r & 3);
  else return (((r >> 3) & 3) << 1) | ((r >> 1) & 1);
}
// V^T tile: row d (64 keys = eight 16-byte units), unit u stored at u ^ v_swz(d).
__device__ __forceinline__ int v_swz(int d) { return (d ^ (d >> 3)) & 7; }

struct PfTile {
  int prefix;  // 1: slots [base, base + 64) of the pair's kept list; 0: positions
  int base;
  int valid;   // valid slots in [0, 64]
};

// Tile tau of a work-group's sequence: the ntp prefix tiles (walked from the last one
// down when rev is set), then the band tiles in ascending order.
__device__ __forceinline__ PfTile pf_tile(int tau, int ntp, int nk, int lo64, int hi, int rev) {
  PfTile t;
  if (tau < ntp) {
    t.prefix = 1;
    t.base = (rev ? ntp - 1 - tau : tau) * PF_KT;
    t.valid = min(PF_KT, nk - t.base);
  } else {
    t.prefix = 0;
    t.base = lo64 + (tau - ntp) * PF_KT;
    t.valid = min(PF_KT, hi - t.base);
  }
  return t;
}

// This thread's share of a tile: KG = pf_kg(D) consecutive key slots, 16-byte chunk dc.
template <int D>
struct PfRegs {
  static constexpr int KG = pf_kg(D);
  u32x4 k[KG];
  u32x4 v[KG];
};

// Positions of this thread's slots in a tile (-1: empty slot).  Prefix tiles read
// kept_idx (the pair's kept positions, ascending).
template <int D>
__device__ __forceinline__ void pf_positions(const int* kidx, const PfTile& t, int s0, int (&pos)[pf_kg(D)]) {
#pragma unroll
  for (int r = 0; r < pf_kg(D); ++r) {
    const int slot = s0 + r;
    if (slot < t.valid) pos[r] = t.prefix ? kidx[t.base + slot] : t.base + slot;
    else pos[r] = -1;
  }
}

template <int D>
__device__ __forceinline__ void pf_load(const uint16_t* kp, const uint16_t* vp, int dc,
                                        const int (&pos)[pf_kg(D)], PfRegs<D>& R) {
#pragma unroll
  for (int r = 0; r < pf_kg(D); ++r) {
    if (pos[r] >= 0) {
      const int64_t off = (int64_t)pos[r] * D + 8 * dc;
      R.k[r] = *reinterpret_cast<const u32x4*>(kp + off);
      R.v[r] = *reinterpret_cast<const u32x4*>(vp + off);
    } else {
      R.k[r] = u32x4{0u, 0u, 0u, 0u};
      R.v[r] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Registers -> LDS.  K rows keep their layout (swizzled chunk); V is transposed: for
// each of the thread's 8 head-dim elements, its KG keys' values are packed with byte
// permutes into one 8-byte (KG = 4) or 4-byte (KG = 2) LDS write.
template <int D>
__device__ __forceinline__ void pf_store(uint16_t* ks, uint16_t* vt, int dc, int s0, const PfRegs<D>& R) {
  constexpr int KG = pf_kg(D);
#pragma unroll
  for (int r = 0; r < KG; ++r) {
    const int row = s0 + r;
    *reinterpret_cast<u32x4*>(ks + row * D + 8 * (dc ^ k_swz<D>(row))) = R.k[r];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = 8 * dc + e;
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint16_t* dst = vt + d * PF_KT + 8 * ((s0 >> 3) ^ v_swz(d)) + (s0 & 7);
    if constexpr (KG == 4) {
      u32x2 w;
      w[0] = __builtin_amdgcn_perm(R.v[1][e >> 1], R.v[0][e >> 1], sel);
      w[1] = __builtin_amdgcn_perm(R.v[3][e >> 1], R.v[2][e >> 1], sel);
      *reinterpret_cast<u32x2*>(dst) = w;
    } else if constexpr (KG == 2) {
      *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(R.v[1][e >> 1], R.v[0][e >> 1], sel);
    } else {
      *dst = static_cast<uint16_t>((e & 1) ? (R.v[0][e >> 1] >> 16) : (R.v[0][e >> 1] & 0xffffu));
    }
  }
}

__device__ __forceinline__ uint32_t low_bits(int n) {
  n = max(0, min(8, n));
  return (1u << n) - 1u;
}

template <int D>
__global__ __launch_bounds__(PF_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_attn_kernel(
    PrefillArgs a) {
  constexpr int KG = pf_kg(D);
  constexpr int DC = D / 8;
  // LDS: two buffers of (K tile, V^T tile), then the reduction slots
  extern __shared__ __attribute__((aligned(16))) uint16_t pf_lds[];
  uint16_t* const kbuf[2] = {pf_lds, pf_lds + 2 * PF_KT * D};
  uint16_t* const vbuf[2] = {pf_lds + PF_KT * D, pf_lds + 3 * PF_KT * D};
  int* const red = reinterpret_cast<int*>(pf_lds + 4 * PF_KT * D);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, G = lane >> 4;
  // Work-group -> (pair, block).  Work-groups are dispatched round-robin over the 8
  // XCDs (blockIdx % 8); an XCD's work-groups are taken in runs of PF_GS (one per CU),
  // each run = PF_GS adjacent position blocks of one pair, so the blocks that read the
  // same kept keys at the same time sit on one XCD and share them through its L2.  An
  // XCD runs all runs of one pair, heavy-first (the last position blocks see the most
  // keys), before the next pair, and consecutive runs walk the kept prefix in opposite
  // directions: a run starts on the keys the previous run read last, which its L2 still
  // holds.  Pair slots enumerate batch rows fastest: the kept fraction varies from head
  // to head (one threshold for all), and an XCD must not inherit one head's load.
  const int x = blockIdx.x % a.nx, k = blockIdx.x / a.nx;
  const int grp = k / PF_GS, j = k % PF_GS;
  const int runs = (a.nblk + PF_GS - 1) / PF_GS;
  const int pi = grp / runs, bgi = grp % runs;
  const int rev = bgi & 1;
  const int blk_raw = bgi * PF_GS + j;
  if (blk_raw >= a.nblk) return;  // padding of the last run (uniform per work-group)
  const int slot = pi * a.nx + x;
  const int B = a.num_pairs / a.Hkv;
  const int b = slot % B, h = slot / B;
  const int pair = b * a.Hkv + h;
  const int blk = a.nblk - 1 - blk_raw;
  const int T = a.T;
  const int i0 = blk * a.pb;
  const int lo64 = max(0, i0 - a.window + 1) & ~(PF_KT - 1);
  const int hi = min(T, i0 + a.pb);

  // kept keys below lo64: popcount of the keep words [0, lo64 / 32)
  const uint32_t* kb = a.keep_bits + (int64_t)pair * a.words;
  int cnt = 0;
  for (int w = tid; w < lo64 / 32; w += PF_THREADS) cnt += __builtin_popcount(kb[w]);
  cnt = wave_sum_i(cnt);
  if (lane == 0) red[wid] = cnt;
  __syncthreads();
  int nk = 0;
#pragma unroll
  for (int w = 0; w < PF_WAVES; ++w) nk += red[w];
  nk = __builtin_amdgcn_readfirstlane(nk);
  const int ntp = (nk + PF_KT - 1) / PF_KT;
  const int ntiles = ntp + (hi - lo64 + PF_KT - 1) / PF_KT;

  const int64_t kv_row0 = (int64_t)pair * T;
  const uint16_t* kp = a.k + kv_row0 * D;
  const uint16_t* vp = a.v + kv_row0 * D;
  const int* kidx = a.kept_idx + kv_row0;
  const int dc = tid % DC, s0 = KG * (tid / DC);

  // this lane's two query rows (column tiles): head and position
  int hq[2], qi[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r0 = 32 * wid + 16 * c;
    hq[c] = h * a.g + r0 / a.pb;
    qi[c] = i0 + r0 % a.pb + n;
  }
  bf16x8 qf[2][D / 32];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint16_t* qrow = a.q + (((int64_t)b * a.Hq + hq[c]) * T + qi[c]) * D;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qi[c] < T) x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qrow + 8 * (4 * kk + G)));
      qf[c][kk] = as_bf16x8(x);
    }
  }

  f32x4 o[D / 16][2];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) o[t][0] = o[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Softmax reference per column (uniform across the column's four lanes): mraw (raw
  // score units, -inf until the column sees a key), mc = mraw * c (0 while mraw is
  // -inf), mlim = mraw + headroom.  Probabilities are exp2(s c - mc); the reference
  // moves only when a score passes mlim, so p <= 2^PF_HEADROOM and the common step
  // needs no cross-lane maximum.
  const float c = a.scale_log2, hr = PF_HEADROOM / c;
  float mraw[2] = {neg_inf(), neg_inf()}, mc[2] = {0.f, 0.f}, mlim[2] = {neg_inf(), neg_inf()};
  float l[2] = {0.f, 0.f};

  // Pipeline: two register sets and two LDS buffers.  A tile's K/V rows are requested
  // three tiles ahead of their use (into the register set of their parity), stored to
  // LDS buffer tau % 2 one tile ahead, and the kept_idx entries are read one tile before
  // the rows.  One barrier per tile: the buffer a step stores into was last read in the
  // step before the previous barrier.
  PfRegs<D> R0, R1;
  int pos[KG];
  pf_positions<D>(kidx, pf_tile(0, ntp, nk, lo64, hi, rev), s0, pos);
  pf_load<D>(kp, vp, dc, pos, R0);
  if (ntiles > 1) {
    pf_positions<D>(kidx, pf_tile(1, ntp, nk, lo64, hi, rev), s0, pos);
    pf_load<D>(kp, vp, dc, pos, R1);
  }
  pf_store<D>(kbuf[0], vbuf[0], dc, s0, R0);
  if (ntiles > 2) {
    pf_positions<D>(kidx, pf_tile(2, ntp, nk, lo64, hi, rev), s0, pos);
    pf_load<D>(kp, vp, dc, pos, R0);
    if (ntiles > 3) pf_positions<D>(kidx, pf_tile(3, ntp, nk, lo64, hi, rev), s0, pos);
  }
  __syncthreads();

  const int slotA = 8 * (n >> 2) + (n & 3);
  // Rn holds tile tau + 1 (when there is one)
  auto step = [&](int tau, PfRegs<D>& Rn) {
    const PfTile tl = pf_tile(tau, ntp, nk, lo64, hi, rev);
    if (tau + 1 < ntiles) {
      pf_store<D>(kbuf[(tau + 1) & 1], vbuf[(tau + 1) & 1], dc, s0, Rn);
      if (tau + 3 < ntiles) {
        pf_load<D>(kp, vp, dc, pos, Rn);
        if (tau + 4 < ntiles) pf_positions<D>(kidx, pf_tile(tau + 4, ntp, nk, lo64, hi, rev), s0, pos);
      }
    }
    const uint16_t* const ks = kbuf[tau & 1];
    const uint16_t* const vt = vbuf[tau & 1];

    uint32_t kw[2] = {0u, 0u};
    if (!tl.prefix) {
      const int w0 = tl.base >> 5;
      kw[0] = kb[w0];
      kw[1] = (w0 + 1 < a.words) ? kb[w0 + 1] : 0u;
    }

#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      if (PF_KT / 2 * ch >= tl.valid) break;
      // S^T for both column tiles
      const int ra = PF_KT / 2 * ch + slotA, rb = ra + 4;
      f32x4 sA[2], sB[2];
      sA[0] = sA[1] = sB[0] = sB[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const int cc = 4 * kk + G;
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + ra * D + 8 * (cc ^ k_swz<D>(ra))));
        const bf16x8 kb8 = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + rb * D + 8 * (cc ^ k_swz<D>(rb))));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          sA[c] = mfma16x16x32(ka, qf[c][kk], sA[c]);
          sB[c] = mfma16x16x32(kb8, qf[c][kk], sB[c]);
        }
      }

      // visibility of this lane's 8 keys (slots 32 ch + 8 G + e) for each column tile
      const int e0 = PF_KT / 2 * ch + 8 * G;
      uint32_t vis[2];
      bool full = false;
      if (tl.prefix) {
        vis[0] = vis[1] = low_bits(tl.valid - e0);
        full = tl.valid == PF_KT;
      } else {
        const uint32_t keep8 = (kw[ch] >> (8 * G)) & 0xffu;
        const int j0 = tl.base + e0;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t causal = low_bits(qi[c] - j0 + 1);
          const uint32_t win = 0xffu & ~low_bits(qi[c] - a.window + 1 - j0);
          vis[c] = causal & (keep8 | win);
        }
      }

      // probabilities of both column tiles, then O^T += V^T P^T with each V^T fragment
      // read from LDS once for both
      bf16x8 phi[2], plo[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        float sv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sv[e] = sA[cc][e];
          sv[e + 4] = sB[cc][e];
        }
        if (!full) {
#pragma unroll
          for (int e = 0; e < 8; ++e) sv[e] = ((vis[cc] >> e) & 1u) ? sv[e] : neg_inf();
        }
        float lm = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        if (__ballot(lm > mlim[cc]) != 0) {
          // some score passed its column's headroom: move the references to the column
          // maxima and rescale what was accumulated against the old ones
          lm = fmaxf(lm, __shfl_xor(lm, 16));
          lm = fmaxf(lm, __shfl_xor(lm, 32));
          const bool upd = lm > mraw[cc];
          const float mcn = lm * c;
          const float alpha = !upd ? 1.0f : (mraw[cc] == neg_inf() ? 0.0f : __builtin_amdgcn_exp2f(mc[cc] - mcn));
          if (upd) {
            mraw[cc] = lm;
            mc[cc] = mcn;
            mlim[cc] = lm + hr;
          }
          l[cc] *= alpha;
          if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
            for (int t = 0; t < D / 16; ++t) o[t][cc] *= alpha;
          }
        }
        float p[8], psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], c, -mc[cc]));
          psum += p[e];
        }
        l[cc] += psum;
        u32x4 ph, pl;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const u32x2 hl = split_bf16x2(p[2 * w], p[2 * w + 1]);
          ph[w] = hl[0];
          pl[w] = hl[1];
        }
        phi[cc] = as_bf16x8(ph);
        plo[cc] = as_bf16x8(pl);
      }
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const int d = 16 * t + n;
        const bf16x8 vf =
            as_bf16x8(*reinterpret_cast<const u32x4*>(vt + d * PF_KT + 8 * ((4 * ch + G) ^ v_swz(d))));
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          o[t][cc] = mfma16x16x32(vf, phi[cc], o[t][cc]);
          o[t][cc] = mfma16x16x32(vf, plo[cc], o[t][cc]);
        }
      }
    }
    __syncthreads();
  };
  for (int tau = 0; tau < ntiles; tau += 2) {
    step(tau, R1);
    if (tau + 1 < ntiles) step(tau + 1, R0);
  }

  // Normalise and store.  Lane (n, G) holds d = 16 t + 4 G + (0..3) of row n of its
  // column tile; the tile's 16 rows are consecutive positions of one head, i.e. one
  // contiguous 16 x D block of the output.  Each wave passes the block through its own
  // LDS rows (padded by 16 bytes against bank conflicts) and writes it as whole lines
  // with non-temporal stores, which keeps the outputs out of L2 (where the kept keys are
  // shared) without the partial-line writes of storing the MFMA layout directly.
  constexpr int OSTR = D * 4 + 16;  // bytes per staged row
  char* const ost = reinterpret_cast<char*>(pf_lds) + wid * 16 * OSTR;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float lt = l[c];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
      *reinterpret_cast<f32x4*>(ost + n * OSTR + (16 * t + 4 * G) * 4) = o[t][c] * inv;
    __syncthreads();
    const int r0 = 32 * wid + 16 * c;
    const int qrow0 = i0 + r0 % a.pb;  // position of row 0 of the block
    float* const oblk = a.out + (((int64_t)b * a.Hq + hq[c]) * T + qrow0) * D;
#pragma unroll
    for (int i = 0; i < 16 * D * 4 / 1024; ++i) {
      const int k = lane + 64 * i;  // 16-byte chunk of the block
      const int row = k / (D / 4), col = k % (D / 4);
      const f32x4 v = *reinterpret_cast<const f32x4*>(ost + row * OSTR + col * 16);
      if (qrow0 + row < T) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(oblk + 4 * k));
    }
    __syncthreads();
  }
}

}  // namespace kvp

using namespace kvp;

kvp_status kvp_launch_prefill_attn(const void* q, const void* k, const void* v, int B, int Hq, int Hkv,
                                   int T, int d, const uint32_t* keep_bits, const int* kept_idx,
                                   int window, float sm_scale, float* out, hipStream_t stream) {
  PrefillArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = out;
  a.keep_bits = keep_bits;
  a.kept_idx = kept_idx;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.T = T;
  a.g = Hq / Hkv;
  a.pb = PF_ROWS / a.g;
  a.nblk = cdiv(T, a.pb);
  a.window = window;
  a.words = cdiv(T, 32);
  a.num_pairs = B * Hkv;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.nx = (a.num_pairs % 8 == 0) ? 8 : 1;
  a.per_x = a.num_pairs / a.nx;
  const int64_t grid = (int64_t)a.nx * a.per_x * cdiv(a.nblk, PF_GS) * PF_GS;
  if (grid > 0x7fffffff) return KVP_E_UNSUPPORTED;
  // tile buffers + reduction slots; at the end each wave stages 16 output rows there
  const size_t lds_tiles = 4 * (size_t)PF_KT * d * sizeof(uint16_t) + PF_WAVES * sizeof(int);
  const size_t lds_out = (size_t)PF_WAVES * 16 * (d * 4 + 16);
  const size_t lds = lds_tiles > lds_out ? lds_tiles : lds_out;
  if (d == 128) prefill_attn_kernel<128><<<(unsigned)grid, PF_THREADS, lds, stream>>>(a);
  else prefill_attn_kernel<64><<<(unsigned)grid, PF_THREADS, lds, stream>>>(a);
  KVP_LAUNCH_CHECK();
  return KVP_OK;
}
