// One unit's attention and summary scan interleaved in a single pass per wave.
//
// Run back to back, the two phases of a unit leave the memory system idle at
// every transition (and the top-K tail of every workgroup lands at the same
// time).  Here each wave streams its attention blocks and its share of the
// summary records together: every step processes one 8 KiB block record and
// SG groups of four 512-byte summary records (SG * 2 KiB), with the next step's
// loads in flight, so the workgroup streams its whole 1.5 MiB without a phase
// change.  Groups left over once the wave's blocks are done go through a
// deeper scan-only loop.  The per-block score arithmetic is the scan path's
// (record_part, row16_sum), so the keys are bit-identical to oasis_score_topk's.
#pragma once

#include "attn_dev.h"
#include "select_dev.h"

namespace oasis {

// Requires at most 64 slots per wave (K <= 256 with one row tile, K <= 128
// with two).  Reads the request's context length from ctx_b (after issuing
// the query and slot-map loads, so that the round trips overlap), writes
// keys[j] for j < nb, returns nb, and ends with the attention merge (so the
// keys are complete in LDS for the whole workgroup afterwards).  `staged`
// runs once the query operands are committed (loads the caller issued before
// the call have completed by then).
template <int D, int RT, int SG, int UL, int TW = RT, bool QL = false, typename Staged>
__device__ __forceinline__ int attn_scan_unit_bf16(const Shape& sh, const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ pool,
                                                   const int32_t* __restrict__ p2l,
                                                   const uint16_t* __restrict__ summ_unit,
                                                   const int32_t* __restrict__ ctx_b, int b, int h,
                                                   float scale_log2, uint16_t* __restrict__ out,
                                                   float* lds, uint32_t* keys,
                                                   Staged&& staged) {
  using AW = AttnWave<D, RT, TW, QL>;
  constexpr int CPL = D / 16;
  constexpr int RW = CPL / 2;          // 32-bit words of one summary row slice
  AW a;
  const int unit = b * sh.H + h;
  // the query operands, the slot map, the context length and the query rows
  // of the group sums are all loaded before the first use of any of them
  a.init_load(sh, q, b, h);
  const int ns = a.n_slots(sh);
  const int j_raw = a.slot_block_raw(sh, p2l, unit, 0, ns);
  const int w = a.w, quad = a.g, n = a.n;
  const int c0 = n * CPL;
  const int L = *ctx_b;
  float Nq[CPL], Pq[CPL];
  // with QL the query operands go to the start of the merge area, which the
  // merge first writes after its own first barrier; the group sums, the same
  // in every wave, are formed by wave 0 alone and passed on after them
  float* sums_lds = lds + AW::QLDS_BYTES / 4;      // [16 lanes][2][CPL]
  if (!QL || w == 0)
  {
    // (a full group of 16 heads, the GQA-16 shape, needs no per-head
    // validity selects: 0.5 us less start-up)
    if (RT == 2 && sh.G == 16)
      group_query_sums<uint16_t, D, CPL, 16, true>(sh, q, 1, b, h, c0, Nq, Pq);
    else
      group_query_sums<uint16_t, D, CPL, (RT == 2 ? 16 : 4)>(sh, q, 1, b, h, c0, Nq, Pq);
  }
  a.init_commit(pool + (size_t)unit * sh.K * AW::REC, lds);
  staged();
  if constexpr (QL) {
    if (w == 0 && quad == 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        sums_lds[n * 2 * CPL + c] = Nq[c];
        sums_lds[n * 2 * CPL + CPL + c] = Pq[c];
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      Nq[c] = sums_lds[n * 2 * CPL + c];
      Pq[c] = sums_lds[n * 2 * CPL + CPL + c];
    }
  }
  const int nb = n_blocks(L, sh.NBmax);
  // record groups: group t of wave w holds records 4*kWaves*t + 4*w + quad
  constexpr int GS = 4 * kWaves;
  const int Gw = nb > 4 * w ? (nb - 4 * w + GS - 1) / GS : 0;

  // Group loads are issued unconditionally (a group past the end loads a
  // clamped in-range record and is ignored): a branch around a load makes
  // the compiler wait for loads issued after it as well.
  using Row = uint32_t __attribute__((ext_vector_type(RW)));
  auto load_groups = [&](int t, int cnt, Row* lo, Row* hi) {
#pragma unroll
    for (int k = 0; k < cnt; ++k) {
      int j = GS * (t + k) + 4 * w + quad;
      j = (t + k < Gw && j < nb) ? j : (nb > 0 ? nb - 1 : 0);
      const uint16_t* rec = summ_unit + (size_t)j * 2 * D + c0;
      lo[k] = __builtin_nontemporal_load(reinterpret_cast<const Row*>(rec));
      hi[k] = __builtin_nontemporal_load(reinterpret_cast<const Row*>(rec + D));
    }
  };
  auto score_groups = [&](int t, int cnt, const Row* lo, const Row* hi) {
#pragma unroll
    for (int k = 0; k < cnt; ++k) {
      if (t + k >= Gw) break;                       // uniform across the wave
      float fl[CPL], fh[CPL];
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        fl[2 * i] = bf16_lo(lo[k][i]); fl[2 * i + 1] = bf16_hi(lo[k][i]);
        fh[2 * i] = bf16_lo(hi[k][i]); fh[2 * i + 1] = bf16_hi(hi[k][i]);
      }
      const float s = row16_sum(record_part<CPL>(fl, fh, Nq, Pq));
      const int j = GS * (t + k) + 4 * w + quad;
      if (n == 0 && j < nb) keys[j] = score_key(s);
    }
  };

  // ---- interleaved steps: one block + SG record groups each ----
  const int nv_l = a.tokens_of(j_raw, sh, L, 0, ns);
  uint64_t todo = ballot(nv_l > 0);
  auto pop = [&]() -> int {
    if (!todo) return -1;
    const int sl = __builtin_ctzll(todo);
    todo &= todo - 1;
    return sl;
  };
  bf16x8 ka[AW::KS], kb[AW::KS];
  i16x4 va[AW::NT], vb[AW::NT];
  Row la[SG], ha[SG], lb[SG], hb[SG];
  int steps = 0;
  int sa = pop();
  if (sa >= 0) {
    a.load(a.slot_of(sa), ka, va);
    load_groups(0, SG, la, ha);
  }
  while (sa >= 0) {
    const int sb = pop();
    if (sb >= 0) {
      a.load(a.slot_of(sb), kb, vb);
      load_groups(SG * (steps + 1), SG, lb, hb);
    }
    a.process(ka, va, __builtin_amdgcn_readlane(nv_l, sa), scale_log2);
    score_groups(SG * steps, SG, la, ha);
    ++steps;
    if (sb < 0) break;
    sa = pop();
    if (sa >= 0) {
      a.load(a.slot_of(sa), ka, va);
      load_groups(SG * (steps + 1), SG, la, ha);
    }
    a.process(kb, vb, __builtin_amdgcn_readlane(nv_l, sb), scale_log2);
    score_groups(SG * steps, SG, lb, hb);
    ++steps;
  }
  // ---- record groups left over: UL at a time ----
  for (int t = SG * steps; t < Gw; t += UL) {
    Row lo[UL], hi[UL];
    load_groups(t, UL, lo, hi);
    score_groups(t, UL, lo, hi);
  }
  a.merge_store(sh, b, h, out, lds);
  return nb;
}

}  // namespace oasis
