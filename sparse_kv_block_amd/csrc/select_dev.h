// Summary scan, top-K selection and capped eviction of one unit (request b,
// KV head h) by one 256-thread workgroup.
//
// Scan (pith.science paper page, "What carries the argument": the draft query
// scans per-block min/max key summaries and ranks every logical block per KV
// head).  The group score of block j is
//     sum_i sum_c max(q_ic * min_jc, q_ic * max_jc),
// which for min <= max equals sum_c [(min+max)/2 * Q_c + (max-min)/2 * A_c]
// with Q_c = sum_i q_ic and A_c = sum_i |q_ic|: two FMAs per channel per block
// instead of 2G.  Sixteen lanes share one 512-byte bf16 summary record (8
// channels each, one 16-byte load of the min row and one of the max row) and
// reduce with DPP inside their 16-lane row; a wave covers 4 blocks per load.
// Summary loads are nontemporal (read once per step).  The scores of the
// unit's whole context stay in LDS as order-preserving 32-bit keys.
//
// Top-K: MSB-first radix bisection on the keys, counting with wave ballots
// (popcount) and one LDS exchange per bit, finds the K-th largest key T; keys
// above T and the lowest-index keys equal to T are compacted and ranked by
// (score desc, block asc).
//
// Capped eviction (same page: admissions per step are capped and each
// admitted block is paired with a least-recently-selected resident block):
// hits are stamped, misses compacted in top-K order with ballots, victims
// (empty slots first, then stale slots by (stamp, block)) ranked by a 64-bit
// key, and the maps updated.
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

// Halved group sums of the query row over the G query heads of KV head h, for
// channels c0 .. c0+CPL: Qh = sum_i q_ic / 2, Ah = sum_i |q_ic| / 2.
template <typename T, int D, int CPL>
__device__ __forceinline__ void group_query_sums(const Shape& sh, const T* __restrict__ q,
                                                 int q_row, int b, int h, int c0, float* Qh,
                                                 float* Ah) {
#pragma unroll
  for (int i = 0; i < CPL; ++i) { Qh[i] = 0.f; Ah[i] = 0.f; }
  for (int i = 0; i < sh.G; ++i) {
    float v[CPL];
    Elem<T>::template load<CPL>(q + ((size_t)(b * 2 + q_row) * sh.Hq + h * sh.G + i) * D + c0, v);
#pragma unroll
    for (int c = 0; c < CPL; ++c) { Qh[c] += v[c]; Ah[c] += fabsf(v[c]); }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) { Qh[c] *= 0.5f; Ah[c] *= 0.5f; }
}

// This lane's part of one block's score (channels of its slice), in the
// channel order every scan path uses, so all of them agree bit for bit.
template <int CPL>
__device__ __forceinline__ float record_part(const float* lo, const float* hi, const float* Qh,
                                             const float* Ah) {
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    s = fmaf(lo[c] + hi[c], Qh[c], s);
    s = fmaf(hi[c] - lo[c], Ah[c], s);
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

  float Qh[CPL], Ah[CPL];
  group_query_sums<T, D, CPL>(sh, q, q_row, b, h, c0, Qh, Ah);

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
      const float s = row16_sum(record_part<CPL>(fl, fh, Qh, Ah));
      const int j = jb + quad + (kThreads / 16) * u;
      if (n == 0 && j < nb) keys[j] = score_key(s);
    }
  }
}

// ---------------------------------------------------------------- top-K
// Most keys one top-K call handles per thread (kMaxKpt * 256 = 8192 blocks).
constexpr int kMaxKpt = 32;
// Scratch `red` (LDS ints): [2][kWaves][4] counts (eviction), four spare
// ints, [2][kMaxKpt][kWaves] compaction counts, then three 256-bin radix
// histograms.
constexpr int kRedHist = 2 * kWaves * 4 + 4 + 2 * kMaxKpt * kWaves;
constexpr int kRedInts = kRedHist + 3 * 256;

// Selects the min(K, nb) best keys; writes sel_idx[0..kk) / sel_key[0..kk) in
// (key desc, index asc) order and returns kk.  cand_* are (K + 4)-entry
// scratch.  Requires nb <= KPT * kThreads.  Thread t holds keys t, t + 256,
// ... in registers for the whole selection.
template <int KPT>
__device__ __forceinline__ int topk_unit(const uint32_t* keys, int nb, int K, int* sel_idx,
                                         uint32_t* sel_key, int* cand_idx, uint32_t* cand_key,
                                         int* red) {
  static_assert(KPT >= 1 && KPT <= kMaxKpt, "keys per thread");
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int kk = K < nb ? K : nb;
  if (kk <= 0) return 0;
  const int act = (nb + kThreads - 1) / kThreads;   // chunks holding keys (uniform)
  uint32_t k[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = i * kThreads + tid;
    k[i] = (i < act && j < nb) ? keys[j] : 0u;
  }
  // 1. K-th largest key T = max{v : #{key >= v} >= kk} by radix selection,
  //    eight bits per round from the top: the keys that match the digits
  //    chosen so far are counted per next digit in an LDS histogram (one
  //    barrier per round); then every wave finds, on its own, the digit at
  //    which the count of larger keys reaches kk.  Three histograms rotate
  //    so that clearing one never races with the use of another.  Key 0 is
  //    never a score key (score_key maps every finite score above it) and
  //    marks the padding.
  int* hist = red + kRedHist;
  const int lane = lane_id();
  hist[tid] = 0;
  hist[kThreads + tid] = 0;
  __syncthreads();
  uint32_t T = 0, mask = 0;
  int rem = kk;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int shift = 24 - 8 * r;
    int* hb = hist + (r % 3) * 256;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (i < act && k[i] != 0u && (k[i] & mask) == T) atomicAdd(&hb[(k[i] >> shift) & 255u], 1);
    __syncthreads();
    // lane l holds digits 255-4l .. 252-4l (descending); inclusive prefix of
    // their counts over the lanes
    const int4 c4 = *reinterpret_cast<const int4*>(hb + 252 - 4 * lane);
    // counts of digits 255-4l, 254-4l, 253-4l, 252-4l
    const int ca = c4.w, cb = c4.z, cc = c4.y, cd = c4.x;
    const int sum = ca + cb + cc + cd;
    int incl = sum;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o);
      incl += lane >= o ? v : 0;
    }
    const int excl = incl - sum;
    const uint64_t cross = ballot(excl < rem && incl >= rem);
    const int L = __builtin_ctzll(cross);
    // within the crossing lane: the digit where the count reaches rem, and
    // the count of larger keys above it
    int above = excl, q = 0;
    if (above + ca < rem) {
      above += ca;
      q = 1;
      if (above + cb < rem) {
        above += cb;
        q = 2;
        if (above + cc < rem) {
          above += cc;
          q = 3;
        }
      }
    }
    const int digit = __shfl(255 - 4 * lane - q, L);
    rem -= __shfl(above, L);
    T |= (uint32_t)digit << shift;
    mask |= 255u << shift;
    hist[((r + 2) % 3) * 256 + tid] = 0;                    // for round r + 2
  }
  // 2. compact in index order (chunk, wave, lane): every key > T, then the
  //    lowest-index keys == T up to kk.  One barrier: each wave publishes its
  //    per-chunk counts, every thread then sums the counts before its own.
  int* cg = red + 2 * kWaves * 4 + 4;
  int* ce = cg + kMaxKpt * kWaves;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (i < act) {
      const int g = __popcll(ballot(k[i] > T));
      const int e = __popcll(ballot(k[i] == T));
      if (lane_id() == 0) { cg[i * kWaves + w] = g; ce[i * kWaves + w] = e; }
    }
  }
  __syncthreads();
  int ngt = 0;
  for (int x = 0; x < act * kWaves; ++x) ngt += cg[x];
  const int need = kk - ngt;
  int run_g = 0, run_e = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (i < act) {
      int og = run_g, oe = run_e;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const int g = cg[i * kWaves + v], e = ce[i * kWaves + v];
        og += v < w ? g : 0;
        oe += v < w ? e : 0;
        run_g += g;
        run_e += e;
      }
      const bool gt = k[i] > T, eq = k[i] == T;
      const uint64_t mg = ballot(gt), me = ballot(eq);
      const int j = i * kThreads + tid;
      if (gt) {
        const int pos = og + lanes_below(mg);
        cand_idx[pos] = j;
        cand_key[pos] = k[i];
      }
      if (eq) {
        const int r = oe + lanes_below(me);
        if (r < need) {
          cand_idx[ngt + r] = j;
          cand_key[ngt + r] = T;
        }
      }
    }
  }
  // pad to a multiple of 4 so the ranking can read four entries at a time
  if (tid < ((kk + 3) & ~3) - kk) {
    cand_key[kk + tid] = 0u;
    cand_idx[kk + tid] = 0x7FFFFFFF;
  }
  __syncthreads();
  // 3. rank the kk candidates by (key desc, index asc).  Up to 128
  //    candidates: two threads per candidate, each over half of the list.
  const int kk4 = (kk + 3) >> 2;
  auto rank_range = [&](uint32_t key, int j, int p0, int p1) {
    int rank = 0;
#pragma unroll 4
    for (int p = p0; p < p1; ++p) {
      const u32x4 kp = reinterpret_cast<const u32x4*>(cand_key)[p];
      const u32x4 jp = reinterpret_cast<const u32x4*>(cand_idx)[p];
#pragma unroll
      for (int e = 0; e < 4; ++e) rank += (kp[e] > key) || (kp[e] == key && (int)jp[e] < j);
    }
    return rank;
  };
  if (kk <= kThreads / 2) {
    const int c = tid % (kThreads / 2), half = tid / (kThreads / 2);
    const int h4 = (kk4 + 1) >> 1;
    int rank = 0;
    uint32_t key = 0;
    int j = 0;
    if (c < kk) {
      key = cand_key[c];
      j = cand_idx[c];
      rank = half ? rank_range(key, j, h4, kk4) : rank_range(key, j, 0, h4);
    }
    if (half && c < kk) cg[c] = rank;                 // compaction counts are spent
    __syncthreads();
    if (!half && c < kk) {
      rank += cg[c];
      sel_idx[rank] = j;
      sel_key[rank] = key;
    }
  } else if (tid < kk) {
    const uint32_t key = cand_key[tid];
    const int j = cand_idx[tid];
    const int rank = rank_range(key, j, 0, kk4);
    sel_idx[rank] = j;
    sel_key[rank] = key;
  }
  __syncthreads();
  return kk;
}

// ---------------------------------------------------------------- capped eviction
struct EvictScratch {
  int* p2l_s;      // [K]
  int* ls_s;       // [K]
  int* miss;       // [K]
  int* victim;     // [K]
  uint64_t* vkey;  // [K]
  int* red;        // [kRedInts]
};

// T: the unit's top-K list in LDS or global memory ([K], -1 = unused entry).
// Pointers l2p/p2l/ls/admit are the unit's slices.
__device__ __forceinline__ void evict_unit(const int* T, int K, int NBmax, int step,
                                           int max_admit, int32_t* __restrict__ l2p,
                                           int32_t* __restrict__ p2l, int32_t* __restrict__ ls,
                                           int32_t* __restrict__ admit,
                                           int32_t* __restrict__ admit_count,
                                           const EvictScratch& x) {
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  if (tid < K) {
    x.p2l_s[tid] = p2l[tid];
    x.ls_s[tid] = ls[tid];
  }
  __syncthreads();
  // 1. stamp resident members of T; flag the missing ones
  const int j = tid < K ? T[tid] : -1;
  const bool valid = j >= 0 && j < NBmax;
  const int s = valid ? l2p[j] : -1;
  const bool hit = valid && s >= 0 && s < K;
  const bool miss = valid && !hit;
  if (hit) x.ls_s[s] = step;
  const uint64_t mm = ballot(miss);
  if (lane_id() == 0) x.red[w] = __popcll(mm);
  __syncthreads();
  int off = 0, nM = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    off += v < w ? x.red[v] : 0;
    nM += x.red[v];
  }
  if (miss) x.miss[off + lanes_below(mm)] = j;
  // 2. victim keys: empty slots by slot, then stale slots by (stamp, block)
  uint64_t key = ~0ull;
  if (tid < K) {
    const int e = x.p2l_s[tid];
    const int st = x.ls_s[tid];
    if (e < 0)
      key = (uint64_t)tid;
    else if (st < step)
      key = (1ull << 63) | ((uint64_t)((uint32_t)st ^ 0x80000000u) << 31) | (uint64_t)(uint32_t)e;
    x.vkey[tid] = key;
  }
  const bool elig = key != ~0ull;
  const uint64_t me = ballot(elig);
  if (lane_id() == 0) x.red[kWaves + w] = __popcll(me);
  __syncthreads();
  int nV = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) nV += x.red[kWaves + v];
  int a = max_admit < nM ? max_admit : nM;
  a = a < nV ? a : nV;
  a = a < 0 ? 0 : a;
  if (tid < ((K + 1) & ~1) - K) x.vkey[K + tid] = ~0ull;   // pad to an even count
  __syncthreads();
  // rank every eligible key among all K: P threads per candidate, each over
  // 1/P of the list (all four waves busy), partial counts summed through LDS
  {
    const int P = K <= kThreads / 4 ? 4 : (K <= kThreads / 2 ? 2 : 1);
    const int span = kThreads / P;
    const int c = tid % span, part = tid / span;
    const int K2 = (K + 1) >> 1;
    const int p0 = part * K2 / P, p1 = (part + 1) * K2 / P;
    int rank = 0;
    uint64_t ck = ~0ull;
    if (c < K) {
      ck = x.vkey[c];
#pragma unroll 8
      for (int p = p0; p < p1; ++p) {
        const u32x4 v = reinterpret_cast<const u32x4*>(x.vkey)[p];
        const uint64_t a0 = ((uint64_t)v[1] << 32) | v[0];
        const uint64_t a1 = ((uint64_t)v[3] << 32) | v[2];
        rank += (a0 < ck) + (a1 < ck);
      }
    }
    int* prt = x.red + kRedHist;                       // the radix histograms are free here
    if (part > 0 && c < K) prt[(part - 1) * span + c] = rank;
    __syncthreads();
    if (part == 0 && c < K && ck != ~0ull) {
      for (int q = 1; q < P; ++q) rank += prt[(q - 1) * span + c];
      if (rank < a) x.victim[rank] = c;
    }
  }
  __syncthreads();
  // 3. apply
  if (tid < a) {
    const int sv = x.victim[tid];
    const int old = x.p2l_s[sv];
    const int aj = x.miss[tid];
    if (old >= 0 && old < NBmax) l2p[old] = -1;
    l2p[aj] = sv;
    x.p2l_s[sv] = aj;
    x.ls_s[sv] = step;
    admit[3 * tid + 0] = aj;
    admit[3 * tid + 1] = sv;
    admit[3 * tid + 2] = old;
  } else if (tid < K) {
    admit[3 * tid + 0] = -1;
    admit[3 * tid + 1] = -1;
    admit[3 * tid + 2] = -1;
  }
  __syncthreads();
  if (tid < K) {
    p2l[tid] = x.p2l_s[tid];
    ls[tid] = x.ls_s[tid];
  }
  if (tid == 0) *admit_count = a;
}

// LDS layout of the select phase (scan keys + top-K + eviction), in bytes.
struct SelectLds {
  int keys, cand_idx, cand_key, sel_idx, sel_key, p2l_s, ls_s, miss, victim, vkey, red, total;
  __host__ __device__ SelectLds(int NBmax, int K) {
    int o = 0;
    auto take = [&](int bytes) { int r = o; o += (bytes + 15) & ~15; return r; };
    keys = take(NBmax * 4);
    cand_idx = take((K + 4) * 4);
    cand_key = take((K + 4) * 4);
    sel_idx = take(K * 4);
    sel_key = take(K * 4);
    p2l_s = take(K * 4);
    ls_s = take(K * 4);
    miss = take(K * 4);
    victim = take(K * 4);
    vkey = take((K + 2) * 8);
    red = take(kRedInts * 4);
    total = o;
  }
};

}  // namespace oasis
