// Summary scan, top-K selection and capped eviction of one unit (request b,
// KV head h) by one 256-thread workgroup.
//
// Scan (pith.science paper page, "What carries the argument": the draft query
// scans per-block min/max key summaries and ranks every logical block per KV
// head).  The group score of block j is
//     sum_i sum_c max(q_ic * min_jc, q_ic * max_jc),
// which for min <= max equals sum_c [min_jc * N_c + max_jc * P_c] with
// N_c = sum_i min(q_ic, 0) and P_c = sum_i max(q_ic, 0): two FMAs per channel
// per block instead of 2G.  Sixteen lanes share one 512-byte bf16 summary record (8
// channels each, one 16-byte load of the min row and one of the max row) and
// reduce with DPP inside their 16-lane row; a wave covers 4 blocks per load.
// Summary loads are nontemporal (read once per step).  The scores of the
// unit's whole context stay in LDS as order-preserving 32-bit keys.
//
// Top-K: radix selection on the keys (eight bits per round, from the highest
// bit on which the keys differ) finds the K-th largest key T; keys above T
// and the lowest-index keys equal to T are compacted and ranked by
// (score desc, block asc).
//
// Capped eviction (same page: admissions per step are capped and each
// admitted block is paired with a least-recently-selected resident block):
// hits are stamped, misses compacted in top-K order with ballots, victims
// (empty slots first, then stale slots by (stamp, block)) ranked by a 64-bit
// key, and the maps updated.  Residency is read from the slot map alone (LDS
// bitmaps of the slots' blocks and of the top-K's), so no l2p entry is read.
#pragma once

#include "common.h"

namespace oasis {

// ---------------------------------------------------------------- summary scan
template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
  // load n consecutive bf16 values (n = 4 or 8) as fp32
  template <int N>
  __device__ static __forceinline__ void load(const uint16_t* p, float* v) {
    if constexpr (N == 8) {
      const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
    } else {
      const u32x2 w = *reinterpret_cast<const u32x2*>(p);
#pragma unroll
      for (int i = 0; i < 2; ++i) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
    }
  }
  __device__ static __forceinline__ float one(const uint16_t* p) { return bf16_bits_to_f32(*p); }
};
template <>
struct Elem<float> {
  template <int N>
  __device__ static __forceinline__ void load(const float* p, float* v) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(p + i);
      v[i] = w[0]; v[i + 1] = w[1]; v[i + 2] = w[2]; v[i + 3] = w[3];
    }
  }
  __device__ static __forceinline__ float one(const float* p) { return *p; }
};

// N consecutive elements held as raw 32-bit words: loaded with nontemporal
// vector loads, unpacked to fp32 later.  Hot loops issue all their loads
// first, unconditionally (out-of-range items load a clamped, in-range
// address and are ignored afterwards), and unpack after: no branch and no
// use sits between a load and the loads issued after it, so the compiler's
// wait counts stay exact and the loads stay in flight together.
template <typename T, int N>
struct Raw {
  static constexpr int W = N * (int)sizeof(T) / 4;
  static_assert(W == 2 || W % 4 == 0, "16- or 8-byte vectors");
  uint32_t w[W];
  __device__ __forceinline__ void load(const T* p) {
    if constexpr (W == 2) {
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
      w[0] = v[0];
      w[1] = v[1];
    } else {
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + i);
        w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
      }
    }
  }
  __device__ __forceinline__ void unpack(float* v) const {
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if constexpr (sizeof(T) == 2) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
      } else {
        v[i] = __uint_as_float(w[i]);
      }
    }
  }
};

// Sign-split group sums of the query row over the G query heads of KV head h,
// for channels c0 .. c0+CPL: Nq = sum_i min(q_ic, 0), Pq = sum_i max(q_ic, 0).
// With min_c <= max_c, max(q min_c, q max_c) = min(q, 0) min_c + max(q, 0) max_c,
// so the group's summed Quest bound is sum_c (Nq_c min_c + Pq_c max_c).
// KB query heads' rows in flight at a time (a load-then-add loop waits a full
// round trip per head), kept as raw words until summed in head order.  The
// interleaved step with two row tiles takes all of up to 16 heads (every
// supported group) in one round trip; the other paths four at a time (the
// raw words of 16 heads would cost the split step a wave per SIMD, and the
// one-tile step measured slower with 8 or 16).  FULL: G is a multiple of KB,
// so no row past G needs its select.
template <typename T, int D, int CPL, int KB = 4, bool FULL = false>
__device__ __forceinline__ void group_query_sums(const Shape& sh, const T* __restrict__ q,
                                                 int q_row, int b, int h, int c0, float* Nq,
                                                 float* Pq) {
#pragma unroll
  for (int i = 0; i < CPL; ++i) { Nq[i] = 0.f; Pq[i] = 0.f; }
  const T* q0 = q + ((size_t)(b * 2 + q_row) * sh.Hq + h * sh.G) * D + c0;
  for (int i0 = 0; i0 < sh.G; i0 += KB) {
    Raw<T, CPL> r[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int i = i0 + k < sh.G ? i0 + k : sh.G - 1;    // clamped, ignored past G
      r[k].load(q0 + (size_t)i * D);
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const bool in = FULL || i0 + k < sh.G;    // a select, not a branch: the loads stay together
      float v[CPL];
      r[k].unpack(v);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        Nq[c] = in ? Nq[c] + fminf(v[c], 0.f) : Nq[c];
        Pq[c] = in ? Pq[c] + fmaxf(v[c], 0.f) : Pq[c];
      }
    }
  }
}

// This lane's part of one block's score (channels of its slice), in the
// channel order every scan path uses, so all of them agree bit for bit.
template <int CPL>
__device__ __forceinline__ float record_part(const float* lo, const float* hi, const float* Nq,
                                             const float* Pq) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    s = fmaf(lo[c], Nq[c], s);
    s = fmaf(hi[c], Pq[c], s);
  }
  return s;
}

// Writes keys[j] for j < nb.  summ_unit points at the unit's [NBmax][2][D].
// U = summary records in flight per 16-lane group (registers vs. bytes in flight).
// Wave w scans the records 16t + 4w + quad (t = 0, 1, ...), quad = lane / 16.
template <typename T, int D, int U>
__device__ __forceinline__ void scan_unit(const Shape& sh, const T* __restrict__ q, int q_row,
                                          const T* __restrict__ summ_unit, int b, int h, int nb,
                                          uint32_t* keys) {
  constexpr int CPL = D / 16;   // channels per lane
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid % kWave;
  const int quad = lane >> 4;
  const int n = lane & 15;
  const int c0 = n * CPL;

  float Nq[CPL], Pq[CPL];
  group_query_sums<T, D, CPL>(sh, q, q_row, b, h, c0, Nq, Pq);

  const T* last = summ_unit + (size_t)(nb > 0 ? nb - 1 : 0) * 2 * D + c0;
  for (int jb = w * 4; jb < nb; jb += kThreads / 16 * U) {
    Raw<T, CPL> lo[U], hi[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + quad + (kThreads / 16) * u;
      const T* rec = j < nb ? summ_unit + (size_t)j * 2 * D + c0 : last;
      lo[u].load(rec);
      hi[u].load(rec + D);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float fl[CPL], fh[CPL];
      lo[u].unpack(fl);
      hi[u].unpack(fh);
      const float s = row16_sum(record_part<CPL>(fl, fh, Nq, Pq));
      const int j = jb + quad + (kThreads / 16) * u;
      if (n == 0 && j < nb) keys[j] = score_key(s);
    }
  }
}

// ---------------------------------------------------------------- top-K
// Most keys one top-K call handles per thread (kMaxKpt * 256 = 8192 blocks).
constexpr int kMaxKpt = 32;
// Scratch `red` (LDS ints): [2][kWaves][4] counts (eviction; the top-K
// exchanges its per-wave OR reductions there), four spare ints,
// [2][kMaxKpt][kWaves] top-K compaction counts (then its partial ranks), then
// four 256-bin radix histograms (one per round), the round-0 digits' bucket
// fill counters and bucket offsets.
constexpr int kRedHist = 2 * kWaves * 4 + 4 + 2 * kMaxKpt * kWaves;
constexpr int kRedInts = kRedHist + 6 * 256;

// Selects the min(K, nb) best keys; writes sel_idx[0..kk) / sel_key[0..kk) in
// (key desc, index asc) order and returns kk.  cand_idx / cand64 are
// (K + 4)-entry scratch.  Requires nb <= KPT * kThreads.  Thread t holds keys
// t, t + kThreads, ... in registers for the whole selection.
//
// 1. The K-th largest key T: the bits all keys share are found first (wave
//    OR reductions of the keys and of their complements); then radix
//    selection eight bits at a time from the highest differing bit: the keys
//    that match the digits chosen so far are counted per next digit in an
//    LDS histogram (one barrier per round; the four histograms are cleared
//    up front) and every wave finds, on its own, the digit at which the count
//    of larger keys reaches kk (a DPP prefix sum over 4 digits per lane).
//    When the chosen digit's count equals the number still needed, every key
//    at or above the prefix is selected and the search stops early with no
//    ties.  Key 0 is never a score key (score_key maps every finite score
//    above it) and marks the padding.
// 2. No ties (the usual case): the kk selected keys are bucketed by their
//    round-0 digit (each bucket's offset is the count of keys in higher
//    digits, from that round's prefix sums; a slot inside the bucket from an
//    LDS counter) and each is ranked only against its own bucket by the
//    packed (key, ~index), so that an entry compares against a few others
//    instead of all kk.
// 3. Ties at T: compaction in index order (chunk, wave, lane) from one packed
//    (above, tied) count per chunk and wave: keys above T go to the
//    candidates, the lowest-index ties straight to the end of the sorted
//    list; then every candidate is ranked against all of them (2-4 threads
//    per candidate, each over a part of the list) by the packed
//    (key, ~index).
template <int KPT>
__device__ __forceinline__ int topk_unit(const uint32_t* keys, int nb, int K, int* sel_idx,
                                         uint32_t* sel_key, int* cand_idx, uint64_t* cand64,
                                         int* red) {
  static_assert(KPT >= 1 && KPT <= kMaxKpt, "keys per thread");
  static_assert(kThreads == 256, "one int4 of histogram per thread to clear");
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = lane_id();
  const int kk = K < nb ? K : nb;
  if (kk <= 0) return 0;
  const int act = (nb + kThreads - 1) / kThreads;
  uint32_t k[KPT];
  uint32_t kor = 0u, knand = 0u;       // OR of the keys, OR of their complements
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = i * kThreads + tid;
    k[i] = (i < act && j < nb) ? keys[j] : 0u;
    if (k[i] != 0u) { kor |= k[i]; knand |= ~k[i]; }
  }
  // the bits every key shares need no radix round
  int* hist = red + kRedHist;                          // [4][256]
  int* fill = hist + 4 * 256;                          // [256]
  int* boff = fill + 256;                              // [256]
  int* xw = red;                                       // [2][kWaves]: the eviction's counters
  reinterpret_cast<int4*>(hist)[tid] = int4{0, 0, 0, 0};
  fill[tid] = 0;
  {
    const uint32_t o = wave_or(kor), n = wave_or(knand);
    if (lane == 0) { xw[w] = (int)o; xw[kWaves + w] = (int)n; }
  }
  __syncthreads();
  uint32_t allor = 0u, allnand = 0u;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) { allor |= (uint32_t)xw[v]; allnand |= (uint32_t)xw[kWaves + v]; }
  const uint32_t diff = allor & allnand;               // bits that differ between keys
  const int hb = diff ? 31 - __builtin_clz(diff) : -1; // highest differing bit
  uint32_t mask = hb < 0 ? ~0u : (hb >= 31 ? 0u : ~((2u << hb) - 1u));
  uint32_t T = allor & mask;
  int rem = kk;
  bool ge = false;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int shift = hb - 7 - 8 * r;                  // digit bits shift+7 .. shift (may be < 0)
    if (shift + 7 < 0) break;
    int* hbuf = hist + r * 256;
    const uint32_t dm = shift >= 0 ? (255u << shift) : (255u >> -shift);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      if (i < act) {
        const bool m = k[i] != 0u && (k[i] & mask) == T;
        const int d = (int)(shift >= 0 ? (k[i] >> shift) & 255u : (k[i] << -shift) & 255u);
        if (m) atomicAdd(&hbuf[d], 1);
      }
    }
    __syncthreads();
    const int4 c4 = *reinterpret_cast<const int4*>(hbuf + 252 - 4 * lane);
    const int ca = c4.w, cb = c4.z, cc = c4.y, cd = c4.x;
    const int sum = ca + cb + cc + cd;
    const int incl = wave_incl_sum(sum);
    const int excl = incl - sum;
    // round 0: each digit's bucket offset (keys in higher digits); every wave
    // writes the same values, so no barrier is needed before its own reads
    if (r == 0)
      *reinterpret_cast<int4*>(boff + 252 - 4 * lane) =
          int4{excl + ca + cb + cc, excl + ca + cb, excl + ca, excl};
    const uint64_t cross = ballot(excl < rem && incl >= rem);
    const int L = __builtin_ctzll(cross);
    int above = excl, q = 0, cq = ca;
    if (above + ca < rem) {
      above += ca; q = 1; cq = cb;
      if (above + cb < rem) {
        above += cb; q = 2; cq = cc;
        if (above + cc < rem) {
          above += cc; q = 3; cq = cd;
        }
      }
    }
    const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane(255 - 4 * lane - q, L);
    rem -= __builtin_amdgcn_readlane(above, L);
    const int cnt = __builtin_amdgcn_readlane(cq, L);
    T |= shift >= 0 ? digit << shift : digit >> -shift;
    mask |= dm;
    if (cnt == rem) {            // every key with this prefix is selected
      ge = true;
      break;
    }
  }
  if (ge) {
    // 2. the kk keys >= T, bucketed by round-0 digit, ranked inside their bucket
    const int shift0 = hb - 7;
    auto digit0 = [&](uint32_t x) -> int {
      return (int)(shift0 >= 0 ? (x >> shift0) & 255u : (x << -shift0) & 255u);
    };
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      if (i < act && k[i] >= T && k[i] != 0u) {
        const int j = i * kThreads + tid;
        const int d = digit0(k[i]);
        const int pos = boff[d] + atomicAdd(&fill[d], 1);
        cand_idx[pos] = j;
        cand64[pos] = ((uint64_t)k[i] << 32) | (uint32_t)~j;
      }
    }
    if (tid == 0) cand64[kk] = 0ull;             // pads a pair read; never ranks above
    __syncthreads();
    if (tid < kk) {
      const uint64_t v = cand64[tid];
      const uint32_t key = (uint32_t)(v >> 32);
      const int d = digit0(key);
      const int b0 = boff[d];
      const int b1 = min(b0 + hist[d], kk);           // the bucket (round 0's counts)
      int rank = b0;
      // pairs of entries; the entries of the pair outside [b0, b1) are skipped
      for (int p = b0 >> 1; 2 * p < b1; ++p) {
        const u32x4 x = reinterpret_cast<const u32x4*>(cand64)[p];
        const uint64_t a0 = ((uint64_t)x[1] << 32) | x[0];
        const uint64_t a1 = ((uint64_t)x[3] << 32) | x[2];
        rank += (2 * p >= b0 && a0 > v) + (2 * p + 1 < b1 && a1 > v);
      }
      sel_idx[rank] = cand_idx[tid];
      sel_key[rank] = key;
    }
    __syncthreads();
    return kk;
  }
  // 3. ties at T: ordered compaction
  int* cnt = red + 2 * kWaves * 4 + 4;
  uint64_t mgv[KPT], mev[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    mgv[i] = 0; mev[i] = 0;
    if (i < act) {
      mgv[i] = ballot(k[i] > T);
      mev[i] = ballot(k[i] == T);
    }
  }
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (i < act && lane == 0) cnt[i * kWaves + w] = (int)((uint32_t)__popcll(mgv[i]) | ((uint32_t)__popcll(mev[i]) << 16));
  __syncthreads();
  constexpr int NP = (KPT * kWaves + 63) / 64;
  const int nx = act * kWaves;
  int ex[NP];
  int carry = 0;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int x = p * 64 + lane;
    const int c = x < nx ? cnt[x] : 0;
    const int in = wave_incl_sum(c) + carry;
    ex[p] = in - c;
    carry = __builtin_amdgcn_readlane(in, 63);
  }
  const int ngt = carry & 0xFFFF;
  const int need = kk - ngt;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (i < act) {
      const int o = __builtin_amdgcn_readlane(ex[(i * kWaves) / 64], (i * kWaves) % 64 + w);
      const int j = i * kThreads + tid;
      if ((mgv[i] >> lane) & 1ull) {
        const int pos = (o & 0xFFFF) + lanes_below(mgv[i]);
        cand_idx[pos] = j;
        cand64[pos] = ((uint64_t)k[i] << 32) | (uint32_t)~j;
      }
      if ((mev[i] >> lane) & 1ull) {
        const int rr = (o >> 16) + lanes_below(mev[i]);
        if (rr < need) {
          sel_idx[ngt + rr] = j;
          sel_key[ngt + rr] = T;
        }
      }
    }
  }
  if (tid == 0) cand64[ngt] = 0ull;            // padding never ranks above a key
  __syncthreads();
  // rank the ngt keys above the threshold: P parts of kThreads / P threads
  // (whole waves), each over 1/P of the list, partial counts summed in LDS
  constexpr int kLogThreads = __builtin_ctz(kThreads);
  const int lp = ngt <= kThreads / 4 ? 2 : (ngt <= kThreads / 2 ? 1 : 0);   // log2 of the parts
  const int P = 1 << lp;
  const int span = kThreads >> lp;
  const int c = tid & (span - 1), part = tid >> (kLogThreads - lp);
  const int n2 = (ngt + 1) >> 1;
  const int p0 = (part * n2) >> lp, p1 = ((part + 1) * n2) >> lp;
  const uint64_t v = c < ngt ? cand64[c] : ~0ull;
  int rank = 0;
#pragma unroll 8
  for (int p = p0; p < p1; ++p) {
    const u32x4 x = reinterpret_cast<const u32x4*>(cand64)[p];
    const uint64_t a0 = ((uint64_t)x[1] << 32) | x[0];
    const uint64_t a1 = ((uint64_t)x[3] << 32) | x[2];
    rank += (a0 > v) + (a1 > v);
  }
  if (P > 1) {
    if (part > 0 && c < ngt) cnt[(part - 1) * span + c] = rank;   // compaction counts are spent
    __syncthreads();
    if (part == 0 && c < ngt)
      for (int q = 1; q < P; ++q) rank += cnt[(q - 1) * span + c];
  }
  if (part == 0 && c < ngt) {
    sel_idx[rank] = cand_idx[c];
    sel_key[rank] = (uint32_t)(v >> 32);
  }
  __syncthreads();
  return kk;
}


// ---------------------------------------------------------------- capped eviction
struct EvictScratch {
  int* p2l_s;      // [K]  the unit's slot map, staged
  int* ls_s;       // [K]  its last-selected stamps, staged
  int* miss;       // [K]
  uint64_t* vkey;  // [K + 2]
  uint32_t* bits;  // [2][kMaxBlocks / 32]: blocks held by a slot, blocks of T
  int* red;        // [kRedInts]
};

__host__ __device__ inline int bitmap_words(int NBmax) { return (NBmax + 31) >> 5; }

// Staging of the eviction's inputs: thread t < K loads slot t's block and
// stamp (evict_load, unconditional clamped loads), then writes them to LDS and
// clears the bitmaps (evict_commit).  At least one barrier must separate the
// commit from evict_unit.
struct EvictStage {
  int e, st;
};
__device__ __forceinline__ EvictStage evict_load(int K, const int32_t* __restrict__ p2l,
                                                 const int32_t* __restrict__ ls) {
  const int t = threadIdx.x < K ? threadIdx.x : K - 1;
  return EvictStage{p2l[t], ls[t]};
}
__device__ __forceinline__ void evict_commit(int K, int NBmax, EvictStage v,
                                             const EvictScratch& x) {
  const int tid = threadIdx.x;
  if (tid < K) {
    x.p2l_s[tid] = v.e;
    x.ls_s[tid] = v.st;
  }
  for (int i = tid; i < 2 * bitmap_words(NBmax); i += kThreads) x.bits[i] = 0u;
}

// T: the unit's top-K list in LDS or global memory ([K], -1 = unused entry).
// Pointers l2p/p2l/ls/admit are the unit's slices; p2l and ls as staged by
// evict_commit.  l2p and p2l are mutual inverses, so block j is resident
// exactly when some slot's p2l entry is j: one bit per block held by a slot,
// one per block of T, and each side tests the other's bits.  Thread t < K
// then acts for slot t: its stamp, its victim key, and, when it is evicted,
// its map updates and admission record.
__device__ __forceinline__ void evict_unit(const int* T, int K, int NBmax, int step,
                                           int max_admit, int32_t* __restrict__ l2p,
                                           int32_t* __restrict__ p2l, int32_t* __restrict__ ls,
                                           int32_t* __restrict__ admit,
                                           int32_t* __restrict__ admit_count,
                                           const EvictScratch& x) {
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  uint32_t* held_bits = x.bits;
  uint32_t* sel_bits = x.bits + bitmap_words(NBmax);
  // 1. membership bits
  const int j = tid < K ? T[tid] : -1;
  const bool valid = j >= 0 && j < NBmax;
  const int e = tid < K ? x.p2l_s[tid] : -1;
  int st = tid < K ? x.ls_s[tid] : 0;
  const bool held = e >= 0 && e < NBmax;
  if (valid) atomicOr(&sel_bits[j >> 5], 1u << (j & 31));
  if (held) atomicOr(&held_bits[e >> 5], 1u << (e & 31));
  __syncthreads();
  // 2. misses of T; stamps of the slots whose block is in T; victim keys:
  //    empty slots by slot, then stale slots by (stamp, block)
  const bool miss = valid && !((held_bits[j >> 5] >> (j & 31)) & 1u);
  if (held && ((sel_bits[e >> 5] >> (e & 31)) & 1u)) st = step;
  uint64_t key = ~0ull;
  if (tid < K) {
    if (e < 0)
      key = (uint64_t)tid;
    else if (st < step)
      key = (1ull << 63) | ((uint64_t)((uint32_t)st ^ 0x80000000u) << 31) | (uint64_t)(uint32_t)e;
    x.vkey[tid] = key;
  }
  if (tid < ((K + 1) & ~1) - K) x.vkey[K + tid] = ~0ull;   // pad to an even count
  const uint64_t mm = ballot(miss);
  const uint64_t me = ballot(key != ~0ull);
  if (lane_id() == 0) {
    x.red[w] = __popcll(mm);
    x.red[kWaves + w] = __popcll(me);
  }
  __syncthreads();
  int off = 0, nM = 0, nV = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    off += v < w ? x.red[v] : 0;
    nM += x.red[v];
    nV += x.red[kWaves + v];
  }
  int a = max_admit < nM ? max_admit : nM;
  a = a < nV ? a : nV;
  a = a < 0 ? 0 : a;                       // the same in every thread
  int rank = a;                            // slot tid's victim rank; >= a: kept
  if (a > 0) {
    if (miss) x.miss[off + lanes_below(mm)] = j;
    // 3. rank every eligible key among all K: P threads per key, each over
    //    1/P of the list (every wave busy), partial counts summed through LDS
    const int lp = K <= kThreads / 4 ? 2 : (K <= kThreads / 2 ? 1 : 0);   // log2 of P
    const int P = 1 << lp;
    const int span = kThreads >> lp;
    const int c = tid & (span - 1), part = tid >> (__builtin_ctz(kThreads) - lp);
    const int K2 = (K + 1) >> 1;
    const int p0 = (part * K2) >> lp, p1 = ((part + 1) * K2) >> lp;
    int r = 0;
    const uint64_t ck = c < K ? x.vkey[c] : ~0ull;
    if (c < K) {
#pragma unroll 8
      for (int p = p0; p < p1; ++p) {
        const u32x4 v = reinterpret_cast<const u32x4*>(x.vkey)[p];
        const uint64_t a0 = ((uint64_t)v[1] << 32) | v[0];
        const uint64_t a1 = ((uint64_t)v[3] << 32) | v[2];
        r += (a0 < ck) + (a1 < ck);
      }
    }
    int* prt = x.red + kRedHist;                       // the radix histograms are free here
    if (part > 0 && c < K) prt[(part - 1) * span + c] = r;
    __syncthreads();                                   // also orders the miss list
    if (part == 0 && c < K && ck != ~0ull) {
      for (int q = 1; q < P; ++q) r += prt[(q - 1) * span + c];
      rank = r;
    }
  }
  // 4. apply: slot tid (tid < K, part 0) takes miss[rank] when rank < a
  if (tid < K) {
    if (rank < a) {
      const int aj = x.miss[rank];
      if (held) l2p[e] = -1;
      l2p[aj] = tid;
      p2l[tid] = aj;
      st = step;
      admit[3 * rank + 0] = aj;
      admit[3 * rank + 1] = tid;
      admit[3 * rank + 2] = e;
    }
    ls[tid] = st;
    if (tid >= a) {
      admit[3 * tid + 0] = -1;
      admit[3 * tid + 1] = -1;
      admit[3 * tid + 2] = -1;
    }
  }
  if (tid == 0) *admit_count = a;
}

// LDS layout of the select phase (scan keys + top-K + eviction), in bytes.
struct SelectLds {
  int keys, cand_idx, cand64, sel_idx, sel_key, p2l_s, ls_s, miss, vkey, bits, red, total;
  __host__ __device__ SelectLds(int NBmax, int K) {
    int o = 0;
    auto take = [&](int bytes) { int r = o; o += (bytes + 15) & ~15; return r; };
    keys = take(NBmax * 4);
    cand_idx = take((K + 4) * 4);
    cand64 = take((K + 4) * 8);
    sel_idx = take(K * 4);
    sel_key = take(K * 4);
    p2l_s = take(K * 4);
    ls_s = take(K * 4);
    miss = take(K * 4);
    vkey = take((K + 2) * 8);
    bits = take(2 * (kMaxBlocks / 32) * 4);
    red = take(kRedInts * 4);
    total = o;
  }
};

}  // namespace oasis
