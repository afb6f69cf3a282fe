// gfx950 kernels of the look-ahead sparse decode step and their launchers.
//
// Every per-unit kernel runs one 256-thread workgroup per (request, KV head):
// the units are independent (their blocks, summaries, maps and slots are
// disjoint).  Only a long context's split over several workgroups hands data
// from one workgroup to another (the scan parts' lists, merged by the last of
// the unit's workgroups to finish).  At batch 128 x 8 KV heads that is 1024
// workgroups; the fused step's register use (about 210 VGPRs, two waves per
// SIMD) places two per CU, so they run in two even rounds over the 256 CUs.
#include <atomic>
#include <mutex>

#include "attn_dev.h"
#include "diag_dev.h"
#include "launch.h"
#include "select_dev.h"
#include "step_dev.h"

namespace oasis {

// ------------------------------------------------------------------ summaries
// Four blocks per wave, one per 16-lane group: lane n of a group takes
// channels n*D/16 .. +D/16 of every token of its block, so each token's key
// row is one contiguous access of the group and the min and max need no lane
// exchanges.  The tokens' loads are issued together (bf16: all 16; fp32: two
// halves of 8, for registers).  A token past the context
// re-reads the last valid one, which leaves min and max unchanged.  The
// records may be host-mapped memory.
constexpr int kSummBlocks = kWaves * 4;   // blocks per workgroup

// W words to p (16- or 8-byte aligned) with nontemporal vector stores.
template <int W, typename T>
__device__ __forceinline__ void store_nt(T* p, const uint32_t* w) {
  static_assert(W == 2 || W % 4 == 0, "8- or 16-byte vectors");
  if constexpr (W == 2) {
    __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2*>(p));
  } else {
#pragma unroll
    for (int i = 0; i < W / 4; ++i)
      __builtin_nontemporal_store(u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]},
                                  reinterpret_cast<u32x4*>(p) + i);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void summarize_kernel(Shape sh, const T* __restrict__ rec,
                                                             const int32_t* __restrict__ ctx,
                                                             T* __restrict__ summ) {
  constexpr int CPL = D / 16;
  constexpr int TB = sizeof(T) == 2 ? kBlock : kBlock / 2;    // tokens per batch of loads
  const int unit = blockIdx.y;
  const int L = ctx[unit / sh.H];
  const int nb = n_blocks(L, sh.NBmax);
  const int lane = threadIdx.x % kWave;
  const int j = blockIdx.x * kSummBlocks + (threadIdx.x / kWave) * 4 + (lane >> 4);
  if (j >= nb) return;
  const int c0 = (lane & 15) * CPL;
  int nv = L - j * kBlock;
  nv = nv > kBlock ? kBlock : nv;
  const T* blk = rec + ((size_t)unit * sh.NBmax + j) * (2 * kBlock * D) + c0;
  float mn[CPL], mx[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) { mn[c] = INFINITY; mx[c] = -INFINITY; }
#pragma unroll
  for (int t0 = 0; t0 < kBlock; t0 += TB) {
    Raw<T, CPL> r[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      const int u = t0 + i;
      r[i].load(blk + (size_t)(u < nv ? u : nv - 1) * D);
    }
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      float v[CPL];
      r[i].unpack(v);
#pragma unroll
      for (int c = 0; c < CPL; ++c) { mn[c] = fminf(mn[c], v[c]); mx[c] = fmaxf(mx[c], v[c]); }
    }
  }
  // nontemporal stores: the summaries are not read again by this launch, and
  // streaming them past the caches keeps the mixed read/write traffic faster
  constexpr int W = CPL * (int)sizeof(T) / 4;
  uint32_t lo[W], hi[W];
#pragma unroll
  for (int i = 0; i < W; ++i) {
    if constexpr (sizeof(T) == 2) {
      lo[i] = f32_to_bf16_bits(mn[2 * i]) | ((uint32_t)f32_to_bf16_bits(mn[2 * i + 1]) << 16);
      hi[i] = f32_to_bf16_bits(mx[2 * i]) | ((uint32_t)f32_to_bf16_bits(mx[2 * i + 1]) << 16);
    } else {
      lo[i] = __float_as_uint(mn[i]);
      hi[i] = __float_as_uint(mx[i]);
    }
  }
  T* out = summ + ((size_t)unit * sh.NBmax + j) * 2 * D + c0;
  store_nt<W>(out, lo);
  store_nt<W>(out + D, hi);
}

// ------------------------------------------------------------------ attention
template <int D, int RT>
__global__ __launch_bounds__(kThreads) void attn_bf16_kernel(Shape sh, const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ pool,
                                                             const int32_t* __restrict__ p2l,
                                                             const int32_t* __restrict__ ctx,
                                                             float scale_log2,
                                                             uint16_t* __restrict__ out) {
  extern __shared__ __align__(16) char smem[];
  const int unit = blockIdx.x;
  const int b = unit / sh.H, h = unit % sh.H;
  attn_unit_bf16<D, RT>(sh, q, pool, p2l, b, h, ctx[b], scale_log2, out,
                        reinterpret_cast<float*>(smem));
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(Shape sh, const float* __restrict__ q,
                                                            const float* __restrict__ pool,
                                                            const int32_t* __restrict__ p2l,
                                                            const int32_t* __restrict__ ctx,
                                                            float scale, float* __restrict__ out) {
  extern __shared__ __align__(16) char smem[];
  const int unit = blockIdx.x;
  const int b = unit / sh.H, h = unit % sh.H;
  attn_unit_f32<D>(sh, q, pool, p2l, b, h, ctx[b], scale, out, reinterpret_cast<float*>(smem));
}

// ------------------------------------------------------------------ scan + top-K
struct SelectPtrs {
  uint32_t* keys;
  int* cand_idx;
  uint64_t* cand64;
  int* sel_idx;
  uint32_t* sel_key;
  EvictScratch ev;
};

__device__ __forceinline__ SelectPtrs select_ptrs(char* smem, int NBmax, int K) {
  SelectLds lay(NBmax, K);
  SelectPtrs p;
  p.keys = reinterpret_cast<uint32_t*>(smem + lay.keys);
  p.cand_idx = reinterpret_cast<int*>(smem + lay.cand_idx);
  p.cand64 = reinterpret_cast<uint64_t*>(smem + lay.cand64);
  p.sel_idx = reinterpret_cast<int*>(smem + lay.sel_idx);
  p.sel_key = reinterpret_cast<uint32_t*>(smem + lay.sel_key);
  p.ev.p2l_s = reinterpret_cast<int*>(smem + lay.p2l_s);
  p.ev.ls_s = reinterpret_cast<int*>(smem + lay.ls_s);
  p.ev.miss = reinterpret_cast<int*>(smem + lay.miss);
  p.ev.vkey = reinterpret_cast<uint64_t*>(smem + lay.vkey);
  p.ev.bits = reinterpret_cast<uint32_t*>(smem + lay.bits);
  p.ev.red = reinterpret_cast<int*>(smem + lay.red);
  return p;
}

// Top-K of the scores in p.keys[0..nb); leaves the sorted list in p.sel_idx
// (entries past kk set to -1) and writes the top-K outputs of the unit.
// KPT: keys per thread, at least nb / kThreads.
template <int KPT = kMaxKpt>
__device__ __forceinline__ void select_from_keys(const Shape& sh, int unit, int nb,
                                                 int32_t* topk_idx, float* topk_score,
                                                 const SelectPtrs& p) {
  const int kk = topk_unit<KPT>(p.keys, nb, sh.K, p.sel_idx, p.sel_key, p.cand_idx,
                                p.cand64, p.ev.red);
  for (int t = threadIdx.x; t < sh.K; t += kThreads) {
    if (t >= kk) p.sel_idx[t] = -1;
    topk_idx[(size_t)unit * sh.K + t] = t < kk ? p.sel_idx[t] : -1;
    topk_score[(size_t)unit * sh.K + t] = t < kk ? key_score(p.sel_key[t]) : -INFINITY;
  }
  __syncthreads();
}

// Scan + select for one unit; leaves the sorted list in p.sel_idx (entries
// past kk set to -1) and writes the top-K outputs.
template <typename T, int D, int U, int KPT>
__device__ __forceinline__ void select_unit(const Shape& sh, const T* q, int q_row, const T* summ,
                                            int unit, int L, int32_t* topk_idx, float* topk_score,
                                            const SelectPtrs& p) {
  const int b = unit / sh.H, h = unit % sh.H;
  const int nb = n_blocks(L, sh.NBmax);
  scan_unit<T, D, U>(sh, q, q_row, summ + (size_t)unit * sh.NBmax * 2 * D, b, h, nb, p.keys);
  __syncthreads();
  select_from_keys<KPT>(sh, unit, nb, topk_idx, topk_score, p);
}

// KPT = keys per thread of the top-K, chosen per launch from NBmax (the
// selection's passes run over every register slot, filled or not).
template <typename T, int D, int KPT>
__global__ __launch_bounds__(kThreads) void score_topk_kernel(Shape sh, const T* __restrict__ q,
                                                              int q_row, const T* __restrict__ summ,
                                                              const int32_t* __restrict__ ctx,
                                                              int32_t* __restrict__ topk_idx,
                                                              float* __restrict__ topk_score) {
  extern __shared__ __align__(16) char smem[];
  const int unit = blockIdx.x;
  const SelectPtrs p = select_ptrs(smem, sh.NBmax, sh.K);
  select_unit<T, D, 4, KPT>(sh, q, q_row, summ, unit, ctx[unit / sh.H], topk_idx, topk_score, p);
}

// ---- hand-over of a split unit's lists inside one launch ----
// A scan part's list goes to the workspace with device-coherent stores, and
// the unit's workgroups then count their arrivals on a per-unit word; the
// last one to arrive merges the lists (and, in the fused step, runs the
// eviction).  The lists are read back with device-coherent loads, so no
// device-scope fence is needed: on gfx950 such a fence writes back or
// invalidates a whole XCD's L2 and costs more than the merge launch it would
// save.  The arrival word holds this launch's tag in bits 16..63 and the count
// in bits 0..15; a word with another tag (an earlier launch, or memory never
// written by one) counts as zero, and the last arrival leaves the count at
// zero, so the workspace needs no initialisation and a replayed launch (same
// tag) starts from zero as well.
template <typename V>
__device__ __forceinline__ void ws_store(V* ptr, V v) {
  __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <bool COHERENT, typename V>
__device__ __forceinline__ V ws_load(const V* ptr) {
  if constexpr (COHERENT)
    return __hip_atomic_load(const_cast<V*>(ptr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *ptr;
}

// A scan part's list (slot 1 + part of the unit), all K entries (key 0 past
// the list's length): blocks c0 + local index.
__device__ __forceinline__ void publish_list(const Shape& sh, const StepWorkspace& ws, int unit,
                                             int parts, int part, int c0, int kk,
                                             const SelectPtrs& p) {
  const size_t slot = (size_t)unit * parts + 1 + part;
  for (int t = threadIdx.x; t < sh.K; t += kThreads) {
    ws_store(&ws.key[slot * sh.K + t], t < kk ? p.sel_key[t] : 0u);
    ws_store(&ws.idx[slot * sh.K + t], t < kk ? c0 + p.sel_idx[t] : -1);
  }
}

// The last scan part's keys, unselected (the merge selects over them).
__device__ __forceinline__ void publish_raw(const StepWorkspace& ws, int unit, int len,
                                            const uint32_t* keys) {
  for (int j = threadIdx.x; j < len; j += kThreads)
    ws_store(&ws.raw[(size_t)unit * kScanChunk + j], keys[j]);
}

// Called by every thread of each of the unit's `total` workgroups once its
// stores to the workspace are issued; true in the last one to arrive.
// ONLY_IF_LAST: arrive only when every other workgroup has arrived (one
// exchange that expects exactly that word, in one round trip), else leave the
// word as it is and return false (the caller then publishes and arrives).
// (Starting every arrival with that exchange instead of a load measured 1 us
// slower in the fused step.)
template <bool ONLY_IF_LAST = false>
__device__ __forceinline__ bool arrive_last(const StepWorkspace& ws, int unit, int total,
                                            int* flag) {
  __builtin_amdgcn_s_waitcnt(0);           // this thread's stores have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long* w = ws.arrive + unit;
    unsigned long long old =
        ONLY_IF_LAST ? ws.tag | (unsigned)(total - 1)
                     : __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool last = false;
    for (;;) {                             // ends: a failed exchange means another arrival
      const int c = (old >> 16) == (ws.tag >> 16) ? (int)(old & 0xffffu) : 0;
      last = c + 1 == total;
      if (ONLY_IF_LAST && !last) break;
      const unsigned long long nw = last ? ws.tag : (ws.tag | (unsigned)(c + 1));
      if (__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT))
        break;
      if (ONLY_IF_LAST) { last = false; break; }
    }
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// LDS for a merge's list entries: block indices from its start, keys at its
// end, right below the select area's key array.
__host__ __device__ inline int merge_lds_bytes(int parts, int K) {
  return parts > 1 ? (((parts - 1) * K * 8 + 15) & ~15) : 0;
}

// The merge of a split unit's scan parts (nb blocks): the lists of parts
// 0 .. nlists-1 (each sorted by (key desc, block asc); a part's list holds
// min(K, its blocks) entries, so only the unit's last part can have fewer
// than K) and, RAW, the keys of part nlists, which skipped its own
// selection, concatenated in part order, so equal keys stay in ascending
// block order and the final top-K equals that of one scan over the whole
// context; then the list out and (EVICT) the capped eviction.  The
// concatenated keys end where the select area's key array begins, which
// holds the raw part's keys: LOCAL, this workgroup scanned that part and
// they are there already; otherwise they come from the workspace.
// COHERENT: the lists were written in the same launch.
template <bool EVICT, bool COHERENT>
__device__ __forceinline__ void merge_unit(const Shape& sh, int unit, int nb, int nlists,
                                           bool raw, bool local,
                                           int step, int max_admit,
                                           int32_t* __restrict__ topk_idx,
                                           float* __restrict__ topk_score, int32_t* l2p,
                                           int32_t* p2l, int32_t* last_sel, int32_t* admit,
                                           int32_t* admit_count, int parts,
                                           const StepWorkspace& ws, const SelectPtrs& p,
                                           char* merge_lds) {
  const int tid = threadIdx.x;
  const int lb = nb - (nlists - 1) * kScanChunk;   // blocks of the last list's part
  const int nl = (nlists - 1) * sh.K + min(sh.K, min(lb, kScanChunk));   // list entries
  const int total = nl + (raw ? nb - nlists * kScanChunk : 0);
  uint32_t* mkey = p.keys - nl;
  int* midx = reinterpret_cast<int*>(merge_lds);
  // every entry in one round trip (EVICT: the slot map and stamps with them)
  EvictStage ev{};
  if constexpr (EVICT)
    ev = evict_load(sh.K, p2l + (size_t)unit * sh.K, last_sel + (size_t)unit * sh.K);
  constexpr int kMaxEntries = (kMaxBlocks / kScanChunk - 1) * 256 + kScanChunk;
  constexpr int kPer = (kMaxEntries + kThreads - 1) / kThreads;
  const int nload = local ? nl : total;
  uint32_t kv[kPer];
  int iv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid + i * kThreads;
    kv[i] = 0u;
    iv[i] = 0;
    if (e < nl) {
      const int pp = e / sh.K;
      const size_t sl = ((size_t)unit * parts + 1 + pp) * sh.K + (e - pp * sh.K);
      kv[i] = ws_load<COHERENT>(&ws.key[sl]);
      iv[i] = ws_load<COHERENT>(&ws.idx[sl]);
    } else if (e < nload) {
      kv[i] = ws_load<COHERENT>(&ws.raw[(size_t)unit * kScanChunk + (e - nl)]);
    }
  }
  if constexpr (EVICT) evict_commit(sh.K, sh.NBmax, ev, p.ev);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = tid + i * kThreads;
    if (e < nload) mkey[e] = kv[i];
    if (e < nl) midx[e] = iv[i];
  }
  __syncthreads();
  // keys per thread sized to the entry count (the selection's passes run over
  // every register slot, filled or not; the result does not depend on it)
  int kk;
  if (total <= kThreads)
    kk = topk_unit<1>(mkey, total, sh.K, p.sel_idx, p.sel_key, p.cand_idx, p.cand64, p.ev.red);
  else if (total <= 2 * kThreads)
    kk = topk_unit<2>(mkey, total, sh.K, p.sel_idx, p.sel_key, p.cand_idx, p.cand64, p.ev.red);
  else if (total <= 4 * kThreads)
    kk = topk_unit<4>(mkey, total, sh.K, p.sel_idx, p.sel_key, p.cand_idx, p.cand64, p.ev.red);
  else if (total <= 8 * kThreads)
    kk = topk_unit<8>(mkey, total, sh.K, p.sel_idx, p.sel_key, p.cand_idx, p.cand64, p.ev.red);
  else
    kk = topk_unit<kPer>(mkey, total, sh.K, p.sel_idx, p.sel_key, p.cand_idx, p.cand64,
                         p.ev.red);
  // (K <= kThreads: thread t < K owns list entry t from here on, and the
  // selection ends with a barrier)
  const int ct = nlists * kScanChunk;               // the unselected part's first block
  for (int t = tid; t < sh.K; t += kThreads) {
    const int e = t < kk ? p.sel_idx[t] : -1;
    const int i = e < 0 ? -1 : (e < nl ? midx[e] : ct + (e - nl));
    p.sel_idx[t] = i;
    topk_idx[(size_t)unit * sh.K + t] = i;
    topk_score[(size_t)unit * sh.K + t] = t < kk ? key_score(p.sel_key[t]) : -INFINITY;
  }
  if constexpr (EVICT) {
    evict_unit(p.sel_idx, sh.K, sh.NBmax, step, max_admit, l2p + (size_t)unit * sh.NBmax,
               p2l + (size_t)unit * sh.K, last_sel + (size_t)unit * sh.K,
               admit + (size_t)unit * sh.K * 3, admit_count + unit, p.ev);
  }
}

// Order of the scan workgroups of a launch whose contexts differ in length:
// workgroups start roughly in index order, so the launch should end on its
// shortest work.  Item j (0-based) maps to (unit, scan part sp): first every
// full kScanChunk-block part (part 0 of every unit that has one, then part 1,
// ...), then the shorter last parts, longest first (in 128-block bands, each
// in request order), every request's heads together; a unit whose context
// fits one part has one item.  Every wave computes the same result: one
// ballot per group and 64 requests, twice (the counts, then the pick).
constexpr int kFullGroups = kMaxBlocks / kScanChunk;   // groups of full parts
constexpr int kBandGroups = kScanChunk / 128;          // groups of last parts
constexpr int kScanGroups = kFullGroups + kBandGroups;

// Request bb's scan parts (np), its full parts and its last part's band
// (-1: none).  Requests past the batch have none.
__device__ __forceinline__ void scan_part_info(const Shape& sh, const int32_t* __restrict__ ctx,
                                               int bb, int& np, int& full, int& band) {
  const int nb = bb < sh.B ? n_blocks(ctx[bb], sh.NBmax) : -1;
  np = nb < 0 ? 0 : (nb > kScanChunk ? (nb + kScanChunk - 1) / kScanChunk : 1);
  const int rem = np > 0 ? nb - (np - 1) * kScanChunk : 0;     // blocks of the last part
  full = rem == kScanChunk ? np : (np > 0 ? np - 1 : 0);
  band = (np > 0 && rem < kScanChunk) ? kBandGroups - 1 - (rem > 0 ? (rem - 1) / 128 : 0) : -1;
}

// Requests per group of the map (cnt, one head each), and the launch's items.
__device__ __forceinline__ int scan_counts(const Shape& sh, const int32_t* __restrict__ ctx,
                                           int* cnt) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int g = 0; g < kScanGroups; ++g) cnt[g] = 0;
  for (int c0 = 0; c0 < sh.B; c0 += kWave) {
    int np, full, band;
    scan_part_info(sh, ctx, c0 + lane, np, full, band);
#pragma unroll
    for (int g = 0; g < kFullGroups; ++g) cnt[g] += __builtin_popcountll(ballot(full > g));
#pragma unroll
    for (int q = 0; q < kBandGroups; ++q)
      cnt[kFullGroups + q] += __builtin_popcountll(ballot(band == q));
  }
  int items = 0;
#pragma unroll
  for (int g = 0; g < kScanGroups; ++g) items += cnt[g];
  return items * sh.H;
}

// Item j from the counts; false past the last item.
__device__ __forceinline__ bool scan_pick(const Shape& sh, const int32_t* __restrict__ ctx,
                                          const int* cnt, int j, int& unit, int& sp) {
  const int lane = threadIdx.x & (kWave - 1);
  int g = kScanGroups, k = j;              // (static indices keep cnt in registers)
#pragma unroll
  for (int x = 0; x < kScanGroups; ++x) {
    const int n = cnt[x] * sh.H;
    if (g == kScanGroups) {
      if (k < n) g = x;
      else k -= n;
    }
  }
  if (g == kScanGroups) return false;
  const int h = k % sh.H;
  k /= sh.H;
  for (int c0 = 0; c0 < sh.B; c0 += kWave) {
    int np, full, band;
    scan_part_info(sh, ctx, c0 + lane, np, full, band);
    const bool in = g < kFullGroups ? full > g : band == g - kFullGroups;
    const uint64_t m = ballot(in);
    const int c = __builtin_popcountll(m);
    if (k < c) {
      const uint64_t pick = ballot(in && lanes_below(m) == k);
      const int l = __builtin_ctzll(pick);
      unit = (c0 + l) * sh.H + h;
      sp = g < kFullGroups ? g : __builtin_amdgcn_readlane(np, l) - 1;
      return true;
    }
    k -= c;
  }
  return false;
}

__device__ __forceinline__ bool scan_item(const Shape& sh, const int32_t* __restrict__ ctx, int j,
                                          int& unit, int& sp) {
  int cnt[kScanGroups];
  scan_counts(sh, ctx, cnt);
  return scan_pick(sh, ctx, cnt, j, unit, sp);
}

// Requests up to which the launches take the ordered mapping above (every
// workgroup reads all context lengths once).
constexpr int kOrderedMaxBatch = 256;

// Long contexts (NBmax above one scan part): workgroup (unit, part) scans the
// part's kScanChunk blocks.  A unit whose context fits one part selects its
// top-K here; otherwise every part but the last selects its local top-K and
// publishes it to the workspace (slot 1 + part of the unit, the layout of the
// fused step's split scan), and the last part, dispatched late in the ordered
// map and so usually the last to finish, skips its selection: when every
// other part has arrived it merges its keys with their lists at once, else it
// publishes its keys unselected and the last arrival merges.  Parts past a
// unit's context exit at once.  (512-block parts measured the same: a faster
// scan, a slower merge.)
template <typename T, int D, int U>
__global__ __launch_bounds__(kThreads) void score_part_kernel(Shape sh, const T* __restrict__ q,
                                                              int q_row, const T* __restrict__ summ,
                                                              const int32_t* __restrict__ ctx,
                                                              int32_t* __restrict__ topk_idx,
                                                              float* __restrict__ topk_score,
                                                              int parts, bool ordered,
                                                              StepWorkspace ws) {
  extern __shared__ __align__(16) char smem[];
  const int units = sh.B * sh.H;
  int unit = blockIdx.x % units;
  int part = blockIdx.x / units;
  if (ordered && !scan_item(sh, ctx, blockIdx.x, unit, part)) return;
  const int b = unit / sh.H, h = unit % sh.H;
  const int nb = n_blocks(ctx[b], sh.NBmax);
  const int np = scan_parts(nb);
  if (part >= np) return;
  __shared__ int last;
  const int head = merge_lds_bytes(parts, sh.K);
  const SelectPtrs p = select_ptrs(smem + head, kScanChunk, sh.K);
  const int c0 = part * kScanChunk;
  const int len = nb - c0 < kScanChunk ? nb - c0 : kScanChunk;
  scan_unit<T, D, U>(sh, q, q_row, summ + ((size_t)unit * sh.NBmax + c0) * 2 * D, b, h, len,
                     p.keys);
  __syncthreads();
  if (np == 1) {
    select_from_keys<kScanChunk / kThreads>(sh, unit, len, topk_idx, topk_score, p);
    return;
  }
  const bool tail = part == np - 1;
  if (tail) {
    if (!arrive_last<true>(ws, unit, np, &last)) {
      publish_raw(ws, unit, len, p.keys);
      if (!arrive_last(ws, unit, np, &last)) return;
    }
  } else {
    const int kk = topk_unit<kScanChunk / kThreads>(p.keys, len, sh.K, p.sel_idx, p.sel_key,
                                                     p.cand_idx, p.cand64, p.ev.red);
    publish_list(sh, ws, unit, parts, part, c0, kk, p);
    if (!arrive_last(ws, unit, np, &last)) return;
  }
  merge_unit<false, true>(sh, unit, nb, np - 1, true, tail, 0, 0, topk_idx, topk_score, nullptr,
                          nullptr, nullptr, nullptr, nullptr, parts, ws, p, smem);
}

// ------------------------------------------------------------------ agreement diagnostic
// Exact block scores of one unit from its keys in the full KV, then the same
// top-K as the summary scan's.
constexpr int kExactInFlight = 4;   // blocks per wave in flight (bf16)

template <typename T, int D, int KPT>
__global__ __launch_bounds__(kThreads) void exact_topk_kernel(Shape sh, const T* __restrict__ q,
                                                              int q_row, const T* __restrict__ rec,
                                                              const int32_t* __restrict__ ctx,
                                                              int32_t* __restrict__ topk_idx,
                                                              float* __restrict__ topk_score) {
  extern __shared__ __align__(16) char smem[];
  const int unit = blockIdx.x;
  const SelectPtrs p = select_ptrs(smem, sh.NBmax, sh.K);
  const int b = unit / sh.H, h = unit % sh.H;
  const int L = ctx[b];
  const int nb = n_blocks(L, sh.NBmax);
  const T* rec_unit = rec + (size_t)unit * sh.NBmax * (2 * kBlock * D);
  if constexpr (sizeof(T) == 2)
    exact_scan_bf16<D, kExactInFlight>(sh, q, q_row, rec_unit, b, h, L, nb, p.keys);
  else
    exact_scan_f32<D>(sh, q, q_row, rec_unit, b, h, L, nb, p.keys);
  __syncthreads();
  select_from_keys<KPT>(sh, unit, nb, topk_idx, topk_score, p);
}

// Per unit: entries among the first exact_n of the exact list that lie in
// [0, NBmax), how many of them the predicted list holds, and how many are
// resident by the slot map (-1 without a map).  A bitmap of the predicted blocks lives in LDS; one list entry per
// thread (K <= 256).
__global__ __launch_bounds__(kThreads) void agreement_kernel(Shape sh, const int32_t* __restrict__ pred,
                                                             const int32_t* __restrict__ exact,
                                                             const int32_t* __restrict__ l2p,
                                                             int exact_n,
                                                             int32_t* __restrict__ counts) {
  __shared__ uint32_t bits[kMaxBlocks / 32];
  const int unit = blockIdx.x;
  const int words = (sh.NBmax + 31) / 32;
  for (int i = threadIdx.x; i < words; i += kThreads) bits[i] = 0u;
  __syncthreads();
  const int t = threadIdx.x;
  if (t < sh.K) {
    const int j = pred[(size_t)unit * sh.K + t];
    if (j >= 0 && j < sh.NBmax) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  int j = t < exact_n ? exact[(size_t)unit * sh.K + t] : -1;
  const bool valid = j >= 0 && j < sh.NBmax;
  const bool agree = valid && ((bits[j >> 5] >> (j & 31)) & 1u);
  const bool res = valid && l2p && l2p[(size_t)unit * sh.NBmax + j] >= 0;
  const int n_valid = __syncthreads_count(valid);
  const int n_agree = __syncthreads_count(agree);
  const int n_res = __syncthreads_count(res);
  if (t == 0) {
    counts[(size_t)unit * 3 + 0] = n_valid;
    counts[(size_t)unit * 3 + 1] = n_agree;
    counts[(size_t)unit * 3 + 2] = l2p ? n_res : -1;
  }
}

// ------------------------------------------------------------------ eviction
__global__ __launch_bounds__(kThreads) void evict_kernel(Shape sh, const int32_t* __restrict__ topk_idx,
                                                         int step, int max_admit, int32_t* l2p,
                                                         int32_t* p2l, int32_t* last_sel,
                                                         int32_t* admit, int32_t* admit_count) {
  extern __shared__ __align__(16) char smem[];
  const int unit = blockIdx.x;
  const SelectPtrs p = select_ptrs(smem, 0, sh.K);
  evict_commit(sh.K, sh.NBmax,
               evict_load(sh.K, p2l + (size_t)unit * sh.K, last_sel + (size_t)unit * sh.K), p.ev);
  __syncthreads();
  evict_unit(topk_idx + (size_t)unit * sh.K, sh.K, sh.NBmax, step, max_admit,
             l2p + (size_t)unit * sh.NBmax, p2l + (size_t)unit * sh.K,
             last_sel + (size_t)unit * sh.K, admit + (size_t)unit * sh.K * 3, admit_count + unit,
             p.ev);
}

// ------------------------------------------------------------------ prefetch
// A small grid of workgroups strides over the (unit, admission) items, two
// records per iteration (16-byte loads, all issued before the stores).  The
// host link, not the CUs, bounds this copy.  The grid follows the transfer:
// one workgroup per kGatherItemsPerGroup items, between kGatherMinGroups and
// kGatherMaxGroups.  Reads of host memory slow the fused step running beside
// them (they share the GPU's path to system memory and its address
// translation): with a 12-layer pipeline at one admission per unit, 128
// workgroups made the step 4.21 ms, 32 made it 3.76 ms (against 3.16 ms with
// no copies); when the link binds (six admissions per unit) 128 workgroups
// move the bytes fastest (10.99 ms against 11.59 ms with 32).
// The source may be host-mapped pinned memory (read over the host link).
constexpr int kGatherMinGroups = 32;
constexpr int kGatherMaxGroups = 128;
constexpr int kGatherItemsPerGroup = 32;

__global__ __launch_bounds__(kThreads) void prefetch_gather_kernel(int units, int K, int NBmax,
                                                                   int rec_bytes, int max_admit,
                                                                   const uint8_t* __restrict__ rec,
                                                                   uint8_t* __restrict__ pool,
                                                                   const int32_t* __restrict__ admit,
                                                                   const int32_t* __restrict__ admit_count) {
  const int items = units * max_admit;
  for (int base = blockIdx.x * 2; base < items; base += gridDim.x * 2) {
    const uint8_t* src[2];
    uint8_t* dst[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      src[e] = nullptr;
      dst[e] = nullptr;
      const int item = base + e;
      if (item >= items) continue;
      const int unit = item / max_admit, k = item % max_admit;
      if (k >= admit_count[unit]) continue;
      const int32_t* a = admit + ((size_t)unit * K + k) * 3;
      const int j = a[0], s = a[1];
      if (j < 0 || j >= NBmax || s < 0 || s >= K) continue;
      src[e] = rec + ((size_t)unit * NBmax + j) * rec_bytes;
      dst[e] = pool + ((size_t)unit * K + s) * rec_bytes;
    }
    for (int off = threadIdx.x * 16; off < rec_bytes; off += kThreads * 32) {
      const int off2 = off + kThreads * 16;
      u32x4 v[2][2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (!src[e]) continue;
        v[e][0] = *reinterpret_cast<const u32x4*>(src[e] + off);
        if (off2 < rec_bytes) v[e][1] = *reinterpret_cast<const u32x4*>(src[e] + off2);
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (!dst[e]) continue;
        *reinterpret_cast<u32x4*>(dst[e] + off) = v[e][0];
        if (off2 < rec_bytes) *reinterpret_cast<u32x4*>(dst[e] + off2) = v[e][1];
      }
    }
  }
}

// ------------------------------------------------------------------ decode append
// One workgroup per request: the request's next position t = ctx_len[b] names
// block j = t / 16 and row u = t % 16.  Thread (h, c) writes channel c of the
// new key into key row u and of the new value into value column u of record
// (b, h, j) in the full KV (device or host-mapped), and into the resident
// copy when the slot map holds block j; the block's summary takes the new key
// (the first token of a block sets both bounds, later tokens widen them; a
// tie keeps the stored value).  After a barrier thread 0 grows ctx_len[b], so
// every thread has read the old length first.
__device__ __forceinline__ float elem_f32(uint16_t x) { return bf16_bits_to_f32(x); }
__device__ __forceinline__ float elem_f32(float x) { return x; }

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void append_kernel(Shape sh, const T* __restrict__ k_new,
                                                          const T* __restrict__ v_new,
                                                          T* __restrict__ rec, T* __restrict__ pool,
                                                          const int32_t* __restrict__ l2p,
                                                          T* __restrict__ summ,
                                                          int32_t* __restrict__ ctx) {
  const int b = blockIdx.x;
  const int t = ctx[b];
  const bool ok = t >= 0 && t < sh.NBmax * kBlock;
  if (ok) {
    const int j = t / kBlock, u = t % kBlock;
    for (int i = threadIdx.x; i < sh.H * D; i += kThreads) {
      const int h = i / D, c = i % D;
      const size_t unit = (size_t)b * sh.H + h;
      const T kv = k_new[unit * D + c];
      const T vv = v_new[unit * D + c];
      T* r = rec + (unit * sh.NBmax + j) * (2 * kBlock * D);
      r[u * D + c] = kv;
      r[kBlock * D + c * kBlock + u] = vv;
      if (pool) {
        const int s = l2p[unit * sh.NBmax + j];
        if (s >= 0 && s < sh.K) {
          T* p = pool + (unit * sh.K + s) * (2 * kBlock * D);
          p[u * D + c] = kv;
          p[kBlock * D + c * kBlock + u] = vv;
        }
      }
      T* sm = summ + (unit * sh.NBmax + j) * 2 * D + c;
      if (u == 0) {
        sm[0] = kv;
        sm[D] = kv;
      } else {
        const float x = elem_f32(kv);
        if (x < elem_f32(sm[0])) sm[0] = kv;
        if (x > elem_f32(sm[D])) sm[D] = kv;
      }
    }
  }
  __syncthreads();
  if (ok && threadIdx.x == 0) ctx[b] = t + 1;
}

// ------------------------------------------------------------------ fused layer step
// Every unit runs attention (the resident blocks) and the summary scan +
// top-K; only the eviction must come after both (it rewrites the slot map that
// attention reads).  Half of the workgroups scan first: their compute-only
// top-K phase then overlaps other workgroups' HBM streaming instead of all
// workgroups stalling the memory system at the same moment.  The selector
// alternates between consecutive workgroups of one XCD (workgroups are dealt
// round-robin over the 8 XCDs) and between the workgroups a CU receives.
__device__ __forceinline__ bool scan_first(int unit) { return ((unit >> 3) ^ (unit >> 8)) & 1; }

// Attention merge area, placed before the select area in LDS.
__host__ __device__ constexpr int attn_region(int D, int RT) {
  return (attn_lds_bytes(D, RT) + 15) & ~15;
}

// Launches with long contexts (NBmax above kScanChunk blocks) split every
// unit over several workgroups, short contexts included: part 0 runs the
// attention, part p >= 1 scans blocks [(p-1)*kScanChunk, p*kScanChunk),
// selects its local top-K and publishes it to the workspace (list slot p of
// the unit).  (Running the attention
// interleaved with the first part's scan, as the one-part kernel does,
// measured slower here: the scan-only workgroups then share that kernel's
// register budget, 2 waves per SIMD instead of 3.)  All of the unit's
// workgroups, the attention's included, then count their arrivals; the last
// merges the lists and runs the eviction, which so comes after the unit's
// attention has read the slot map.

// Scan items dispatched ahead of the attention workgroups in an ordered split
// launch (all of them when there are fewer).  Workgroups are served oldest first, so these full-part scans
// finish early and their slots take further scans while the attention
// workgroups stream; the launch then ends on fewer late full-part scans.  On
// 64 requests x 8 KV heads of lognormal contexts (3 workgroups per CU,
// 512 attention workgroups, 1,208 scan items), interleaved in one process:
// 1.3-1.7 us faster at 192, 0.9-1.1 at 128, none at 64, 96, 256 or 768.
constexpr int kScanAhead = 192;

// LDS before the select area: the attention merge area, which also holds a
// split unit's concatenated lists once the attention is done.
__host__ __device__ inline int step_head_bytes(int attn_bytes, int parts, int K) {
  const int m = merge_lds_bytes(parts, K);
  return attn_bytes > m ? attn_bytes : m;
}

template <typename T, int D, int RT, int U, bool IL>
__global__ __launch_bounds__(kThreads) void layer_step_kernel(
    Shape sh, const T* __restrict__ q, const T* __restrict__ pool, const T* __restrict__ summ,
    const int32_t* __restrict__ ctx, float scale, int step, int max_admit, T* __restrict__ out,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_score, int32_t* l2p, int32_t* p2l,
    int32_t* last_sel, int32_t* admit, int32_t* admit_count, int parts, bool ordered,
    int first_fill, StepWorkspace ws) {
  extern __shared__ __align__(16) char smem[];
  constexpr bool kMfma = sizeof(T) == 2;
  const int units = sh.B * sh.H;
  int unit = blockIdx.x % units;
  int slot = blockIdx.x / units;
  int sp = -1;                             // scan part, ordered mapping
  if (!IL && ordered && parts > 1) {
    // dispatch order: the first `ahead` scan items, the attention workgroups,
    // the remaining scan items
    int cnt[kScanGroups];
    const int items = scan_counts(sh, ctx, cnt);
    const int ahead = items < kScanAhead ? items : kScanAhead;
    const int n = blockIdx.x;
    if (n >= ahead && n < ahead + units) {
      slot = 0;
      unit = n - ahead;
    } else {
      slot = 1;
      if (!scan_pick(sh, ctx, cnt, n < ahead ? n : n - units, unit, sp)) return;
    }
  }
  const int b = unit / sh.H, h = unit % sh.H;
  const int tid = threadIdx.x;
  const int head = step_head_bytes(kMfma ? attn_region(D, RT) : attn_f32_lds_bytes(D), parts, sh.K);
  const SelectPtrs p = select_ptrs(smem + head, sh.NBmax < kScanChunk ? sh.NBmax : kScanChunk,
                                   sh.K);
  // the unit's top-K list out, then the capped eviction (kk = list length)
  // (K <= kThreads: thread t < K owns list entry t here and in the eviction,
  // and the selection ends with a barrier)
  auto finish = [&](int kk) {
    for (int t = tid; t < sh.K; t += kThreads) {
      if (t >= kk) p.sel_idx[t] = -1;
      topk_idx[(size_t)unit * sh.K + t] = t < kk ? p.sel_idx[t] : -1;
      topk_score[(size_t)unit * sh.K + t] = t < kk ? key_score(p.sel_key[t]) : -INFINITY;
    }
    evict_unit(p.sel_idx, sh.K, sh.NBmax, step, max_admit, l2p + (size_t)unit * sh.NBmax,
               p2l + (size_t)unit * sh.K, last_sel + (size_t)unit * sh.K,
               admit + (size_t)unit * sh.K * 3, admit_count + unit, p.ev);
  };
  if constexpr (IL && kMfma) {
    // Workgroups past the first fill of the CUs (first_fill resident at once)
    // start as slots free up and end the launch; the CUs serve their waves
    // oldest first, so these take a higher priority against the first
    // fill's stragglers (16K shape: 1.1-1.5 us faster; GQA-16 unchanged).
    if ((int)blockIdx.x >= first_fill) __builtin_amdgcn_s_setprio(2);
    // Launched only when every context fits one scan part (one workgroup per
    // unit): one pass streams the unit's blocks and its summary records
    // together, two summary groups per block step (with 32 rows the query
    // operands sit in LDS so that both groups fit 2 waves per SIMD).  The
    // context length is read inside, after the query and slot-map loads.
    // the eviction's slot map and stamps travel with the query loads
    const EvictStage ev =
        evict_load(sh.K, p2l + (size_t)unit * sh.K, last_sel + (size_t)unit * sh.K);
    const int nb = attn_scan_unit_bf16<D, RT, 2, 8, RT, (RT == 2)>(
        sh, q, pool, p2l, summ + (size_t)unit * sh.NBmax * 2 * D, ctx + b, b, h, scale, out,
        reinterpret_cast<float*>(smem), p.keys, [&]() { evict_commit(sh.K, sh.NBmax, ev, p.ev); });
    __syncthreads();
    finish(topk_unit<kScanChunk / kThreads>(p.keys, nb, sh.K, p.sel_idx, p.sel_key, p.cand_idx,
                                            p.cand64, p.ev.red));
    return;
  }
  const int L = ctx[b];
  const int nb = n_blocks(L, sh.NBmax);
  // a split launch hands every non-empty unit to an attention workgroup and
  // its scan parts (one for a context that fits one part): the longest item
  // is then one attention pass, not attention and scan back to back
  const int active = parts > 1 && nb > 0 ? 1 + scan_parts(nb) : 1;
  // Without the ordered mapping (more than kOrderedMaxBatch requests) a split
  // unit's last (shortest) scan part takes the last slot: workgroups start in
  // slot order, so the launch ends on short workgroups instead of full
  // 1024-block scans started when the first ones drain.
  int part = slot;
  if (sp >= 0)
    part = 1 + sp;
  else if (active > 1 && slot >= 1)
    part = slot == parts - 1 ? active - 1 : (slot < active - 1 ? slot : active);
  if (part >= active) return;
  const bool whole = active == 1;          // one workgroup does the whole unit
  const int c0 = whole ? 0 : (part - 1) * kScanChunk;
  const int len = whole ? nb : (nb - c0 < kScanChunk ? nb - c0 : kScanChunk);

  auto attention = [&]() {
    if constexpr (kMfma)
      attn_unit_bf16<D, RT>(sh, q, pool, p2l, b, h, L, scale, out, reinterpret_cast<float*>(smem));
    else
      attn_unit_f32<D>(sh, q, pool, p2l, b, h, L, scale, out, reinterpret_cast<float*>(smem));
  };
  auto scan_select = [&]() -> int {
    scan_unit<T, D, U>(sh, q, 1, summ + ((size_t)unit * sh.NBmax + c0) * 2 * D, b, h, len, p.keys);
    __syncthreads();
    return topk_unit<kScanChunk / kThreads>(p.keys, len, sh.K, p.sel_idx, p.sel_key, p.cand_idx,
                                            p.cand64, p.ev.red);
  };
  if (!whole) {
    // (Here every scan part selects.  The last part skipping its selection,
    // as in the standalone split scan, measured 0.5-0.7 us slower: a scan
    // part arrives last in every unit, but the launch ends on full-part scans
    // that start when the attention workgroups drain, and the merges that
    // take raw keys cost more.)
    __shared__ int last;
    if (part == 0) {
      attention();
    } else {
      const int kk = scan_select();
      publish_list(sh, ws, unit, parts, part - 1, c0, kk, p);
    }
    if (!arrive_last(ws, unit, active, &last)) return;
    merge_unit<true, true>(sh, unit, nb, active - 1, false, false, step, max_admit, topk_idx,
                           topk_score, l2p, p2l, last_sel, admit, admit_count, parts, ws, p,
                           smem);
    return;
  }
  evict_commit(sh.K, sh.NBmax,
               evict_load(sh.K, p2l + (size_t)unit * sh.K, last_sel + (size_t)unit * sh.K), p.ev);
  int kk;
  if (scan_first(unit)) {
    kk = scan_select();
    attention();
  } else {
    attention();
    kk = scan_select();
  }
  finish(kk);
}

// ------------------------------------------------------------------ dense attention
// The dense comparator: decode attention of both rows over every valid token
// of the full, HBM-resident KV.  Split over the context: workgroup (unit, c)
// runs the same per-wave MFMA core over blocks [c*128, (c+1)*128) and writes
// the unnormalised partial (max, sum, output row) of every row; a second
// kernel merges the partials of a unit.
constexpr int kDenseChunk = 4 * kWave / 2;   // 128 blocks: 32 per wave

template <int D, int RT>
__global__ __launch_bounds__(kThreads) void dense_partial_kernel(Shape sh, const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ rec,
                                                                 const int32_t* __restrict__ ctx,
                                                                 float scale_log2, int chunks,
                                                                 float* __restrict__ part) {
  extern __shared__ __align__(16) char smem[];
  using AW = AttnWave<D, RT, RT>;
  const int units = sh.B * sh.H;
  const int unit = blockIdx.x % units, c = blockIdx.x / units;
  const int b = unit / sh.H, h = unit % sh.H;
  const int L = ctx[b];
  const int nb = n_blocks(L, sh.NBmax);
  const int rows = 2 * sh.G;
  float* mypart = part + ((size_t)unit * chunks + c) * rows * (D + 2);
  const int j0 = c * kDenseChunk;
  if (j0 >= nb) {                                   // nothing in this chunk
    for (int r = threadIdx.x; r < rows; r += kThreads) {
      mypart[(size_t)r * (D + 2)] = -INFINITY;
      mypart[(size_t)r * (D + 2) + 1] = 0.f;
    }
    return;
  }
  AW a;
  a.init(sh, q, rec + (size_t)unit * sh.NBmax * AW::REC, b, h);
  // wave w takes blocks j0 + w, j0 + w + 4, ...: the four waves stream one
  // contiguous region together
  const int lane = threadIdx.x % kWave;
  auto blk = [&](int i) { return j0 + a.w + kWaves * i; };
  int nv_l = 0;
  if (lane < kDenseChunk / kWaves && blk(lane) < nb) {
    const int nv = L - blk(lane) * kBlock;
    nv_l = nv < 0 ? 0 : (nv > kBlock ? kBlock : nv);
  }
  uint64_t todo = ballot(nv_l > 0);
  auto pop = [&]() -> int {
    if (!todo) return -1;
    const int sl = __builtin_ctzll(todo);
    todo &= todo - 1;
    return sl;
  };
  bf16x8 ka[AW::KS], kb[AW::KS];
  i16x4 va[AW::NT], vb[AW::NT];
  int sa = pop();
  if (sa >= 0) a.load(blk(sa), ka, va);
  while (sa >= 0) {
    const int sb = pop();
    if (sb >= 0) a.load(blk(sb), kb, vb);
    a.process(ka, va, __builtin_amdgcn_readlane(nv_l, sa), scale_log2);
    if (sb < 0) break;
    sa = pop();
    if (sa >= 0) a.load(blk(sa), ka, va);
    a.process(kb, vb, __builtin_amdgcn_readlane(nv_l, sb), scale_log2);
  }
  a.merge_store(sh, b, h, nullptr, reinterpret_cast<float*>(smem), mypart);
}

template <int D>
__global__ __launch_bounds__(kThreads) void dense_merge_kernel(Shape sh, int chunks,
                                                               const float* __restrict__ part,
                                                               uint16_t* __restrict__ out) {
  const int unit = blockIdx.x;
  const int b = unit / sh.H, h = unit % sh.H;
  const int G = sh.G, rows = 2 * G;
  const float* up = part + (size_t)unit * chunks * rows * (D + 2);
  for (int e = threadIdx.x; e < rows * D; e += kThreads) {
    const int r = e / D, c = e % D;
    float M = -INFINITY;
    for (int k = 0; k < chunks; ++k) M = fmaxf(M, up[((size_t)k * rows + r) * (D + 2)]);
    float Ls = 0.f, o = 0.f;
    for (int k = 0; k < chunks; ++k) {
      const float* pr = up + ((size_t)k * rows + r) * (D + 2);
      if (pr[0] == -INFINITY) continue;
      const float f = exp2f(pr[0] - M);
      Ls += pr[1] * f;
      o += pr[2 + c] * f;
    }
    const int row = r < G ? 0 : 1;
    const int head = h * G + (r < G ? r : r - G);
    out[((size_t)(b * 2 + row) * sh.Hq + head) * D + c] = f32_to_bf16_bits(Ls > 0.f ? o / Ls : 0.f);
  }
}

// ------------------------------------------------------------------ launchers
namespace {
constexpr float kLog2e = 1.4426950408889634f;

constexpr size_t kMaxLds = 64 * 1024;   // dynamic LDS per workgroup

float scale_or_default(float scale, int d) { return scale > 0.f ? scale : 1.0f / sqrtf((float)d); }

int rt_of(int G) { return 2 * G <= 16 ? 1 : 2; }

// Workgroups of `kernel` (256 threads, `lds` dynamic LDS bytes) resident at
// once on the current device: its CUs times the workgroups one CU holds;
// looked up once per device, kernel and LDS size (a fixed table, no
// allocation).  0 when the runtime cannot tell or the table is full.
int resident_workgroups(const void* kernel, size_t lds) {
  struct Entry { int dev; const void* kernel; size_t lds; int count; };
  static std::mutex mu;
  static Entry table[64];
  static int used = 0;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (table[i].dev == dev && table[i].kernel == kernel && table[i].lds == lds)
      return table[i].count;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, lds) != hipSuccess) {
    (void)hipGetLastError();                // not the launch's error
    return 0;
  }
  if (used == 64) return 0;
  table[used] = Entry{dev, kernel, lds, cus * per_cu};
  return table[used++].count;
}

// A tag for one launch's arrival words: odd in bits 16..63, zero below.
std::atomic<unsigned long long> g_launches{0};
unsigned long long launch_tag() {
  const unsigned long long t = g_launches.fetch_add(1, std::memory_order_relaxed) + 1;
  return ((t << 1) | 1ull) << 16;
}
}  // namespace

hipError_t launch_summarize(const Shape& sh, int dtype, const void* records, const int32_t* ctx,
                            void* summ, hipStream_t st) {
  dim3 grid((sh.NBmax + kSummBlocks - 1) / kSummBlocks, sh.B * sh.H);
  if (dtype == 1) {
    if (sh.d == 128)
      hipLaunchKernelGGL((summarize_kernel<uint16_t, 128>), grid, dim3(kThreads), 0, st, sh,
                         (const uint16_t*)records, ctx, (uint16_t*)summ);
    else
      hipLaunchKernelGGL((summarize_kernel<uint16_t, 64>), grid, dim3(kThreads), 0, st, sh,
                         (const uint16_t*)records, ctx, (uint16_t*)summ);
  } else {
    if (sh.d == 128)
      hipLaunchKernelGGL((summarize_kernel<float, 128>), grid, dim3(kThreads), 0, st, sh,
                         (const float*)records, ctx, (float*)summ);
    else
      hipLaunchKernelGGL((summarize_kernel<float, 64>), grid, dim3(kThreads), 0, st, sh,
                         (const float*)records, ctx, (float*)summ);
  }
  return hipGetLastError();
}

hipError_t launch_attn(const Shape& sh, int dtype, const void* q, const void* pool,
                       const int32_t* p2l, const int32_t* ctx, float scale, void* out,
                       hipStream_t st) {
  const float sc = scale_or_default(scale, sh.d);
  dim3 grid(sh.B * sh.H);
  if (dtype == 1) {
    const int rt = rt_of(sh.G);
    const size_t lds = attn_lds_bytes(sh.d, rt);
    const float sl = sc * kLog2e;
#define OASIS_ATTN(D_, RT_)                                                                   \
  hipLaunchKernelGGL((attn_bf16_kernel<D_, RT_>), grid, dim3(kThreads), lds, st, sh,          \
                     (const uint16_t*)q, (const uint16_t*)pool, p2l, ctx, sl, (uint16_t*)out)
    if (sh.d == 128) { if (rt == 1) OASIS_ATTN(128, 1); else OASIS_ATTN(128, 2); }
    else             { if (rt == 1) OASIS_ATTN(64, 1);  else OASIS_ATTN(64, 2); }
#undef OASIS_ATTN
  } else {
    if (sh.d == 128)
      hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(kThreads), attn_f32_lds_bytes(128), st, sh,
                         (const float*)q, (const float*)pool, p2l, ctx, sc, (float*)out);
    else
      hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(kThreads), attn_f32_lds_bytes(64), st, sh,
                         (const float*)q, (const float*)pool, p2l, ctx, sc, (float*)out);
  }
  return hipGetLastError();
}

hipError_t launch_score_topk(const Shape& sh, int dtype, const void* q, int q_row, const void* summ,
                             const int32_t* ctx, int32_t* topk_idx, float* topk_score,
                             void* workspace, hipStream_t st) {
  const int parts = step_parts(sh.NBmax);
  if (parts > 1) {
    // split over scan parts, then merge the parts' lists
    StepWorkspace ws = step_workspace(workspace, sh.B * sh.H, parts, sh.K);
    ws.tag = launch_tag();
    const size_t lds = merge_lds_bytes(parts, sh.K) + SelectLds(kScanChunk, sh.K).total;
    if (lds > kMaxLds) return hipErrorInvalidConfiguration;
    dim3 pgrid(sh.B * sh.H * scan_parts(sh.NBmax));
#define OASIS_PART(T_, D_)                                                                    \
  hipLaunchKernelGGL((score_part_kernel<T_, D_, 8>), pgrid, dim3(kThreads), lds, st, sh,      \
                     (const T_*)q, q_row, (const T_*)summ, ctx, topk_idx, topk_score, parts,   \
                     sh.B <= kOrderedMaxBatch, ws)
    if (dtype == 1) { if (sh.d == 128) { OASIS_PART(uint16_t, 128); } else { OASIS_PART(uint16_t, 64); } }
    else            { if (sh.d == 128) { OASIS_PART(float, 128); }    else { OASIS_PART(float, 64); } }
#undef OASIS_PART
    return hipGetLastError();
  }
  dim3 grid(sh.B * sh.H);
  const size_t lds = SelectLds(sh.NBmax, sh.K).total;
  const bool small = sh.NBmax <= 4 * kThreads;     // 4 keys per thread suffice
#define OASIS_SCORE(T_, D_)                                                                   \
  if (small)                                                                                  \
    hipLaunchKernelGGL((score_topk_kernel<T_, D_, 4>), grid, dim3(kThreads), lds, st, sh,     \
                       (const T_*)q, q_row, (const T_*)summ, ctx, topk_idx, topk_score);      \
  else                                                                                        \
    hipLaunchKernelGGL((score_topk_kernel<T_, D_, kMaxKpt>), grid, dim3(kThreads), lds, st,   \
                       sh, (const T_*)q, q_row, (const T_*)summ, ctx, topk_idx, topk_score)
  if (dtype == 1) { if (sh.d == 128) { OASIS_SCORE(uint16_t, 128); } else { OASIS_SCORE(uint16_t, 64); } }
  else            { if (sh.d == 128) { OASIS_SCORE(float, 128); }    else { OASIS_SCORE(float, 64); } }
#undef OASIS_SCORE
  return hipGetLastError();
}

hipError_t launch_exact_topk(const Shape& sh, int dtype, const void* q, int q_row,
                             const void* records, const int32_t* ctx, int32_t* topk_idx,
                             float* topk_score, hipStream_t st) {
  dim3 grid(sh.B * sh.H);
  const size_t lds = SelectLds(sh.NBmax, sh.K).total;
  const bool small = sh.NBmax <= 4 * kThreads;     // 4 keys per thread suffice
#define OASIS_EXACT(T_, D_)                                                                   \
  if (small)                                                                                  \
    hipLaunchKernelGGL((exact_topk_kernel<T_, D_, 4>), grid, dim3(kThreads), lds, st, sh,     \
                       (const T_*)q, q_row, (const T_*)records, ctx, topk_idx, topk_score);   \
  else                                                                                        \
    hipLaunchKernelGGL((exact_topk_kernel<T_, D_, kMaxKpt>), grid, dim3(kThreads), lds, st,   \
                       sh, (const T_*)q, q_row, (const T_*)records, ctx, topk_idx, topk_score)
  if (dtype == 1) { if (sh.d == 128) { OASIS_EXACT(uint16_t, 128); } else { OASIS_EXACT(uint16_t, 64); } }
  else            { if (sh.d == 128) { OASIS_EXACT(float, 128); }    else { OASIS_EXACT(float, 64); } }
#undef OASIS_EXACT
  return hipGetLastError();
}

hipError_t launch_agreement(const Shape& sh, const int32_t* pred, const int32_t* exact,
                            const int32_t* l2p, int exact_n, int32_t* counts, hipStream_t st) {
  hipLaunchKernelGGL(agreement_kernel, dim3(sh.B * sh.H), dim3(kThreads), 0, st, sh, pred, exact,
                     l2p, exact_n, counts);
  return hipGetLastError();
}

hipError_t launch_evict(const Shape& sh, const int32_t* topk_idx, int step, int max_admit,
                        int32_t* l2p, int32_t* p2l, int32_t* last_sel, int32_t* admit,
                        int32_t* admit_count, hipStream_t st) {
  const size_t lds = SelectLds(0, sh.K).total;
  hipLaunchKernelGGL(evict_kernel, dim3(sh.B * sh.H), dim3(kThreads), lds, st, sh, topk_idx, step,
                     max_admit, l2p, p2l, last_sel, admit, admit_count);
  return hipGetLastError();
}

hipError_t launch_append(const Shape& sh, int dtype, const void* k_new, const void* v_new,
                         void* records, void* pool, const int32_t* l2p, void* summ,
                         int32_t* ctx, hipStream_t st) {
  dim3 grid(sh.B);
  if (dtype == 1) {
    auto* f = sh.d == 128 ? append_kernel<uint16_t, 128> : append_kernel<uint16_t, 64>;
    hipLaunchKernelGGL(f, grid, dim3(kThreads), 0, st, sh, (const uint16_t*)k_new,
                       (const uint16_t*)v_new, (uint16_t*)records, (uint16_t*)pool, l2p,
                       (uint16_t*)summ, ctx);
  } else {
    auto* f = sh.d == 128 ? append_kernel<float, 128> : append_kernel<float, 64>;
    hipLaunchKernelGGL(f, grid, dim3(kThreads), 0, st, sh, (const float*)k_new,
                       (const float*)v_new, (float*)records, (float*)pool, l2p, (float*)summ,
                       ctx);
  }
  return hipGetLastError();
}

hipError_t launch_prefetch_gather(const Shape& sh, size_t rec_bytes, const void* records, void* pool,
                                  const int32_t* admit, const int32_t* admit_count, int max_admit,
                                  hipStream_t st) {
  if (max_admit <= 0) return hipSuccess;
  const long long items = (long long)sh.B * sh.H * max_admit;
  long long groups = items / kGatherItemsPerGroup;
  groups = groups < kGatherMinGroups ? kGatherMinGroups : (groups > kGatherMaxGroups ? kGatherMaxGroups : groups);
  if (groups > (items + 1) / 2) groups = (items + 1) / 2;      // at least two items per group
  hipLaunchKernelGGL(prefetch_gather_kernel, dim3((unsigned)groups), dim3(kThreads), 0, st, sh.B * sh.H, sh.K,
                     sh.NBmax, (int)rec_bytes, max_admit, (const uint8_t*)records, (uint8_t*)pool,
                     admit, admit_count);
  return hipGetLastError();
}

hipError_t launch_layer_step(const Shape& sh, int dtype, const void* q, const void* pool,
                             const void* summ, const int32_t* ctx, float scale, int step,
                             int max_admit, void* out, int32_t* topk_idx, float* topk_score,
                             int32_t* l2p, int32_t* p2l, int32_t* last_sel, int32_t* admit,
                             int32_t* admit_count, void* workspace, hipStream_t st) {
  const float sc = scale_or_default(scale, sh.d);
  const int parts = step_parts(sh.NBmax);      // list slots per unit (slot 0 unused)
  StepWorkspace ws = step_workspace(workspace, sh.B * sh.H, parts, sh.K);
  ws.tag = launch_tag();
  const bool ordered = sh.B <= kOrderedMaxBatch;
  dim3 grid(sh.B * sh.H * parts);
  const size_t sel = SelectLds(sh.NBmax < kScanChunk ? sh.NBmax : kScanChunk, sh.K).total;
  if (dtype == 1) {
    const int rt = rt_of(sh.G);
    const size_t lds = step_head_bytes(attn_region(sh.d, rt), parts, sh.K) + sel;
    if (lds > kMaxLds) return hipErrorInvalidConfiguration;
    const float sl = sc * kLog2e;
    // One scan part per unit: attention and scan interleaved in one pass (at
    // 2 waves per SIMD; with 32 rows the wave holds both row tiles and takes
    // one summary group per block step).  Split scans: separate phases with
    // a 6-deep scan unroll, which fits 3 waves per SIMD, the better trade
    // when many short workgroups share the CUs.
#define OASIS_STEP(D_, RT_, U_, IL_)                                                            \
  hipLaunchKernelGGL((layer_step_kernel<uint16_t, D_, RT_, U_, IL_>), grid, dim3(kThreads), lds, \
                     st, sh, (const uint16_t*)q, (const uint16_t*)pool, (const uint16_t*)summ,   \
                     ctx, sl, step, max_admit, (uint16_t*)out, topk_idx, topk_score, l2p, p2l,   \
                     last_sel, admit, admit_count, parts, ordered,                               \
                     IL_ ? resident_workgroups(                                                  \
                               (const void*)layer_step_kernel<uint16_t, D_, RT_, U_, IL_>, lds)  \
                         : 0,                                                                    \
                     ws)
    if (parts == 1) {
      if (sh.d == 128) { if (rt == 1) OASIS_STEP(128, 1, 8, true); else OASIS_STEP(128, 2, 8, true); }
      else             { if (rt == 1) OASIS_STEP(64, 1, 8, true);  else OASIS_STEP(64, 2, 8, true); }
    } else {
      if (sh.d == 128) { if (rt == 1) OASIS_STEP(128, 1, 6, false); else OASIS_STEP(128, 2, 6, false); }
      else             { if (rt == 1) OASIS_STEP(64, 1, 6, false);  else OASIS_STEP(64, 2, 6, false); }
    }
#undef OASIS_STEP
  } else {
    const size_t lds = step_head_bytes(attn_f32_lds_bytes(sh.d), parts, sh.K) + sel;
    if (lds > kMaxLds) return hipErrorInvalidConfiguration;
#define OASIS_STEP32(D_)                                                                        \
  hipLaunchKernelGGL((layer_step_kernel<float, D_, 1, 4, false>), grid, dim3(kThreads), lds, st, sh,    \
                     (const float*)q, (const float*)pool, (const float*)summ, ctx, sc, step,     \
                     max_admit, (float*)out, topk_idx, topk_score, l2p, p2l, last_sel, admit,    \
                     admit_count, parts, ordered, 0, ws)
    if (sh.d == 128) OASIS_STEP32(128); else OASIS_STEP32(64);
#undef OASIS_STEP32
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ scratch
// Device memory for the callers that cannot allocate (oasis_layer_step_noalloc):
// the fused step's split-scan lists.  Each device that loads the library holds
// its own copy until the process ends.  Host code never uses the array's name
// as an address: the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_pointer(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t layer_step_workspace_bytes(const Shape& sh) {
  return step_workspace_bytes(sh.B * sh.H, step_parts(sh.NBmax), sh.K);
}

size_t dense_workspace_bytes(const Shape& sh) {
  const int chunks = (sh.NBmax + kDenseChunk - 1) / kDenseChunk;
  return (size_t)sh.B * sh.H * chunks * 2 * sh.G * (sh.d + 2) * sizeof(float);
}

hipError_t launch_dense_attn(const Shape& sh, const void* q, const void* records, const int32_t* ctx,
                             float scale, void* out, void* workspace, hipStream_t st) {
  const float sl = scale_or_default(scale, sh.d) * kLog2e;
  const int chunks = (sh.NBmax + kDenseChunk - 1) / kDenseChunk;
  const int units = sh.B * sh.H;
  const int rt = rt_of(sh.G);
  const size_t lds = attn_lds_bytes(sh.d, rt);
  float* part = static_cast<float*>(workspace);
#define OASIS_DENSE(D_, RT_)                                                                    \
  hipLaunchKernelGGL((dense_partial_kernel<D_, RT_>), dim3(units * chunks), dim3(kThreads), lds, \
                     st, sh, (const uint16_t*)q, (const uint16_t*)records, ctx, sl, chunks, part)
  if (sh.d == 128) { if (rt == 1) OASIS_DENSE(128, 1); else OASIS_DENSE(128, 2); }
  else             { if (rt == 1) OASIS_DENSE(64, 1);  else OASIS_DENSE(64, 2); }
#undef OASIS_DENSE
  if (sh.d == 128)
    hipLaunchKernelGGL(dense_merge_kernel<128>, dim3(units), dim3(kThreads), 0, st, sh, chunks, part,
                       (uint16_t*)out);
  else
    hipLaunchKernelGGL(dense_merge_kernel<64>, dim3(units), dim3(kThreads), 0, st, sh, chunks, part,
                       (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace oasis
