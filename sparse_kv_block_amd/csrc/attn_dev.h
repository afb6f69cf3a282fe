// Look-ahead attention of one unit (request b, KV head h) by one 256-thread
// workgroup.  Both query rows (normal and draft) of the G query heads of the KV
// head are stacked as 2G rows and share every K/V load (pith.science paper
// page, "What carries the argument": one kernel runs the normal and the draft
// token over the same resident set).
//
// bf16 path: CDNA4 MFMA.  Each wave owns a contiguous range of the unit's
// slots and streams their 8 KiB block records straight from HBM into
// registers (no LDS staging: the record layout already matches the operand
// layout, and nontemporal loads keep the once-read stream from churning the
// caches), one block ahead of the math:
//   logits  D[token][row] = K[token][:] . Q[row][:]   mfma 16x16x32 bf16, d/32 steps
//   output  O[c][row]    += V^T[c][token] . P[token][row]  mfma 16x16x16 bf16, d/16 tiles
// The 16x16 logit tile leaves lane (g, n) holding rows n, tokens 4g..4g+3,
// which is exactly the B operand layout of the 16x16x16 P.V step, so P never
// leaves registers.  Softmax is online with a lazy rescale: the running max
// only moves when a block's max exceeds it by more than 8 (in log2 units), so
// unnormalised weights stay below 2^8 and the rescale factor is almost always 1.  The four waves' partial (max, sum, O)
// are merged through LDS at the end.
//
// f32 path: plain VALU (one wave per query row); it serves the small fp32
// workloads whose tolerance is 1e-5.
#pragma once

#include "common.h"

namespace oasis {

// Row stride (floats) of the merge's partial-output buffers: rows of D
// channels padded by 4, so that the 16 rows' 16-byte accesses at one channel
// fall on distinct banks.
__host__ __device__ constexpr int attn_row_stride(int D) { return D + 4; }

// LDS bytes the bf16 attention merge needs (two [16][D + 4] partial-output
// buffers per row tile, per-wave row max and sum, per-row denominators).
__host__ __device__ constexpr int attn_lds_bytes(int D, int RT) {
  return (RT * 2 * 16 * attn_row_stride(D) + kWaves * 16 * RT * 2 + 2 * 16 * RT) * 4;
}

// RT = 16-row tiles of the stacked rows (1: up to 16 rows, 2: up to 32).
// By default every wave holds all RT tiles and the four waves split the
// unit's slots four ways, so each record is fetched once per workgroup.
// With TW = 1 < RT = 2, wave w takes row tile w & 1 and slot half w >> 1
// instead (half the accumulators per wave); the two waves of a slot half then
// read the same records back to back (the second read is a cache hit), so
// those loads keep the default cache policy instead of the streaming one.
// TW = row tiles one wave holds.  TW == RT == 2: every wave takes both tiles
// of its quarter of the slots (each record fetched once per workgroup, twice
// the accumulators per wave).
//
// QL: the query operands, identical in every wave when TW == RT, live once
// per workgroup in LDS (TW * KS * 64 16-byte entries at `qlds`, written by
// wave 0 in init(); the caller puts a barrier between init() and the first
// process()) and each logit MFMA reads its operand from there: 8 * TW VGPRs
// per lane fewer for the same arithmetic.
template <int D, int RT, int TW = 1, bool QL = false>
struct AttnWave {
  static constexpr int KS = D / 32;   // logit MFMA steps
  static constexpr int NT = D / 16;   // output tiles
  static constexpr int REC = 2 * kBlock * D;
  static constexpr bool kPairs = RT == 2 && TW == 1;   // waves paired on a slot half
  static constexpr int NSPLIT = kPairs ? kWaves / 2 : kWaves;
  static_assert(!QL || TW == RT, "LDS query operands need every wave to hold every tile");
  static constexpr int QLDS_BYTES = QL ? TW * KS * kWave * 16 : 0;

  int w, g, n, rt, split;
  bf16x8 qop[QL ? 1 : TW][QL ? 1 : KS];
  const bf16x8* qlds;
  float m_run[TW], l_run[TW];
  f32x4 acc[TW][NT];
  const uint16_t* unit_pool;

  // query operand: lane (g, n) holds row 16*(rt+t) + n, channels 32*kk + 8g .. +8.
  // init_load issues the operand loads (a row past 2G loads row 0 and is
  // zeroed in init_commit), so that callers can issue their other start-up
  // loads before the first wait: with each load inside `if (valid)` and the
  // LDS store after it, the compiler waited a full round trip per operand.
  u32x4 qraw[TW][KS];
  bool qvalid[TW];

  __device__ __forceinline__ void init_load(const Shape& sh, const uint16_t* __restrict__ q, int b,
                                            int h) {
    const int lane = threadIdx.x % kWave;
    w = threadIdx.x / kWave;
    g = lane >> 4;
    n = lane & 15;
    rt = kPairs ? (w & 1) : 0;
    split = kPairs ? (w >> 1) : w;
    const int G = sh.G;
    // with QL only wave 0 needs the operands (it stores them for all)
    if (QL && w != 0) return;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const int r = 16 * (rt + t) + n;
      qvalid[t] = r < 2 * G;
      const int rc = qvalid[t] ? r : 0;
      const int row = rc < G ? 0 : 1;
      const int head = h * G + (rc < G ? rc : rc - G);
      const uint16_t* qr = q + ((size_t)(b * 2 + row) * sh.Hq + head) * D;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        qraw[t][kk] = *reinterpret_cast<const u32x4*>(qr + 32 * kk + 8 * g);
    }
  }

  // unit_base: the unit's first record (slot 0 of its pool, or block 0 of its
  // records for the dense variant).  q_area: QLDS_BYTES of LDS (QL only).
  __device__ __forceinline__ void init_commit(const uint16_t* __restrict__ unit_base,
                                              void* q_area = nullptr) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const bf16x8 v = __builtin_bit_cast(bf16x8, qvalid[t] ? qraw[t][kk] : z);
        if constexpr (QL) {
          if (w == 0) static_cast<bf16x8*>(q_area)[(t * KS + kk) * kWave + lane] = v;
        } else {
          qop[t][kk] = v;
        }
      }
      m_run[t] = -INFINITY;
      l_run[t] = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    unit_pool = unit_base;
    qlds = static_cast<const bf16x8*>(q_area);
  }

  __device__ __forceinline__ void init(const Shape& sh, const uint16_t* __restrict__ q,
                                       const uint16_t* __restrict__ unit_base, int b, int h,
                                       void* q_area = nullptr) {
    init_load(sh, q, b, h);
    init_commit(unit_base, q_area);
  }

  // This wave's slots are split, split + NSPLIT, split + 2*NSPLIT, ...: the
  // waves of a workgroup take consecutive records in turn, so at any moment
  // they stream one contiguous region of the pool rather than NSPLIT separate
  // ones (measured ~5% more HBM bandwidth on gfx950).
  __device__ __forceinline__ int n_slots(const Shape& sh) const {
    return split < sh.K ? (sh.K - split + NSPLIT - 1) / NSPLIT : 0;
  }
  __device__ __forceinline__ int slot_of(int i) const { return split + NSPLIT * i; }

  // Logical block held by this wave's slot number ib + lane, loaded
  // unconditionally (lanes past ie read a clamped slot; tokens_of ignores
  // them), so that the load can be issued long before its use.
  __device__ __forceinline__ int slot_block_raw(const Shape& sh, const int32_t* __restrict__ p2l,
                                                int unit, int ib, int ie) const {
    const int lane = threadIdx.x % kWave;
    int k = ib + lane < ie ? ib + lane : ie - 1;
    k = k < 0 ? 0 : k;
    return p2l[(size_t)unit * sh.K + slot_of(k)];
  }
  // Valid-token count of the slot whose raw block is j (lanes past ie give 0).
  __device__ __forceinline__ int tokens_of(int j, const Shape& sh, int L, int ib, int ie) const {
    const int lane = threadIdx.x % kWave;
    if (lane >= ie - ib || j < 0 || j >= sh.NBmax) return 0;
    const int nv = L - j * kBlock;
    return nv < 0 ? 0 : (nv > kBlock ? kBlock : nv);
  }

  // Valid-token count of this wave's slot number ib + lane (lanes past ie give 0).
  __device__ __forceinline__ int slot_tokens(const Shape& sh, const int32_t* __restrict__ p2l, int unit,
                                             int L, int ib, int ie) const {
    const int lane = threadIdx.x % kWave;
    int nv_l = 0;
    if (lane < ie - ib) {
      const int j = p2l[(size_t)unit * sh.K + slot_of(ib + lane)];
      if (j >= 0 && j < sh.NBmax) {
        const int nv = L - j * kBlock;
        nv_l = nv < 0 ? 0 : (nv > kBlock ? kBlock : nv);
      }
    }
    return nv_l;
  }

  __device__ __forceinline__ void load(int slot, bf16x8* kr, i16x4* vr) const {
    const uint16_t* rec = unit_pool + (size_t)slot * REC;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const bf16x8* pk = reinterpret_cast<const bf16x8*>(rec + n * D + 32 * kk + 8 * g);
      kr[kk] = kPairs ? *pk : __builtin_nontemporal_load(pk);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const i16x4* pv = reinterpret_cast<const i16x4*>(rec + kBlock * D + (16 * nt + n) * kBlock + 4 * g);
      vr[nt] = kPairs ? *pv : __builtin_nontemporal_load(pv);
    }
  }

  __device__ __forceinline__ void process(const bf16x8* kr, const i16x4* vr, int nv, float scale_log2) {
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        bf16x8 qv;
        if constexpr (QL) qv = qlds[(t * KS + kk) * kWave + g * 16 + n];
        else qv = qop[t][kk];
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[kk], qv, z, 0, 0, 0);
      }
      float zz[4];
      float bm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zz[i] = (4 * g + i < nv) ? z[i] * scale_log2 : -INFINITY;
        bm = fmaxf(bm, zz[i]);
      }
      bm = xrow_max(bm);
      // f is 1 unless the block max exceeds the running max by more than 8;
      // the rescale runs only when some row of the wave needs it (rows that
      // do not multiply by 1).
      const bool need = bm > m_run[t] + 8.0f;
      const float f = need ? __builtin_amdgcn_exp2f(m_run[t] - bm) : 1.0f;
      m_run[t] = need ? bm : m_run[t];
      if (ballot(need)) {
        l_run[t] *= f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[t][nt] *= f;
      }
      // weights rounded to bf16 (round to nearest even, v_cvt_pk_bf16_f32)
      // for the P.V product; the denominator sums the rounded weights.  The
      // bare v_exp_f32: a weight below 2^-126 of the running maximum comes
      // out as 0 instead of a denormal
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(zz[i] - m_run[t]);
      const bf16x2 p01 = __builtin_convertvector((f32x2){e[0], e[1]}, bf16x2);
      const bf16x2 p23 = __builtin_convertvector((f32x2){e[2], e[3]}, bf16x2);
      l_run[t] += (float)p01[0];
      l_run[t] += (float)p01[1];
      l_run[t] += (float)p23[0];
      l_run[t] += (float)p23[1];
      const u32x2 pw = {__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
      const i16x4 pb = __builtin_bit_cast(i16x4, pw);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[t][nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vr[nt], pb, acc[t][nt], 0, 0, 0);
    }
  }

  // Merges the waves that share a row tile through LDS and writes the rows:
  // normalised bf16 rows to `out`, or, when `part` is given, the unnormalised
  // partial (running max, sum, output row) of each row to part[r][0 .. D+2).
  // LDS: [2*TW][16][D + 4] partial outputs (row-major: a lane's four
  // accumulator channels are one 16-byte access), [kWaves][16*TW] max and
  // sum, [16*RT] x 2.
  __device__ __forceinline__ void merge_store(const Shape& sh, int b, int h,
                                              uint16_t* __restrict__ out, float* lds,
                                              float* __restrict__ part = nullptr) const {
    const int tid = threadIdx.x;
    const int G = sh.G;
    constexpr int S = attn_row_stride(D);
    float* obuf = lds;                                   // [TW][2][16][S]
    float* mbuf = lds + TW * 2 * 16 * S;                 // [kWaves][16*TW]
    float* lbuf = mbuf + kWaves * 16 * TW;               // [kWaves][16*TW]
    float* lstar = lbuf + kWaves * 16 * TW;              // [16*RT]
    float* mstar = lstar + 16 * RT;                      // [16*RT]
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const float lsum = xrow_sum(l_run[t]);
      if (g == 0) {
        mbuf[(w * TW + t) * 16 + n] = m_run[t];
        lbuf[(w * TW + t) * 16 + n] = lsum;
      }
    }
    __syncthreads();
    float fw[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < kWaves; ++v)
        if (!kPairs || (v & 1) == rt) M = fmaxf(M, mbuf[(v * TW + t) * 16 + n]);
      float Ls = 0.f;
      fw[t] = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        if (kPairs && (v & 1) != rt) continue;
        const float mv = mbuf[(v * TW + t) * 16 + n];
        const float f = (mv == -INFINITY) ? 0.f : exp2f(mv - M);
        Ls += lbuf[(v * TW + t) * 16 + n] * f;
        if (v == w) fw[t] = f;
      }
      if ((kPairs ? w == rt : w == 0) && g == 0) {
        lstar[16 * (rt + t) + n] = Ls;
        mstar[16 * (rt + t) + n] = M;
      }
    }
    // waves 0,1 write their scaled partial outputs into buffer pair slot w&1;
    // waves 2,3 add theirs, then 4,5 and so on.  Paired waves: buffer slot =
    // row tile.
    for (int phase = 0; phase < kWaves / 2; ++phase) {
      if ((w >> 1) == phase) {
#pragma unroll
        for (int t = 0; t < TW; ++t) {
          float* ob = obuf + (t * 2 + (w & 1)) * 16 * S + n * S + 4 * g;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            f32x4* p = reinterpret_cast<f32x4*>(ob + 16 * nt);
            const f32x4 v = acc[t][nt] * fw[t];
            if (phase == 0) *p = v; else *p += v;
          }
        }
      }
      __syncthreads();
    }
    // eight consecutive channels of one row per thread and pass: one 16-byte
    // store of the normalised bf16 row slice
    const int rows = 2 * G;
    constexpr int CV = 8;
    for (int e = tid; e < rows * (D / CV); e += kThreads) {
      const int r = e / (D / CV), c0 = (e % (D / CV)) * CV;
      const int rr = r % 16, tile = r / 16;
      float o[CV];
      {
        const float* s0 = obuf + (kPairs ? tile : tile * 2) * 16 * S + rr * S + c0;
#pragma unroll
        for (int i = 0; i < CV; i += 4) {
          f32x4 v = *reinterpret_cast<const f32x4*>(s0 + i);
          if (!kPairs) v += *reinterpret_cast<const f32x4*>(s0 + 16 * S + i);
#pragma unroll
          for (int k = 0; k < 4; ++k) o[i + k] = v[k];
        }
      }
      const float Ls = lstar[r];
      if (part) {
        float* pr = part + (size_t)r * (D + 2);
        if (c0 == 0) { pr[0] = mstar[r]; pr[1] = Ls; }
#pragma unroll
        for (int i = 0; i < CV; ++i) pr[2 + c0 + i] = o[i];
        continue;
      }
      const int row = r < G ? 0 : 1;
      const int head = h * G + (r < G ? r : r - G);
      u32x4 packed;
#pragma unroll
      for (int i = 0; i < CV / 2; ++i)
        packed[i] = (uint32_t)f32_to_bf16_bits(Ls > 0.f ? o[2 * i] / Ls : 0.f) |
                    ((uint32_t)f32_to_bf16_bits(Ls > 0.f ? o[2 * i + 1] / Ls : 0.f) << 16);
      *reinterpret_cast<u32x4*>(out + ((size_t)(b * 2 + row) * sh.Hq + head) * D + c0) = packed;
    }
  }
};

template <int D, int RT, int TW = RT>
__device__ __forceinline__ void attn_unit_bf16(const Shape& sh, const uint16_t* __restrict__ q,
                                               const uint16_t* __restrict__ pool,
                                               const int32_t* __restrict__ p2l, int b, int h,
                                               int L, float scale_log2,
                                               uint16_t* __restrict__ out, float* lds) {
  using AW = AttnWave<D, RT, TW>;
  AW a;
  const int unit = b * sh.H + h;
  a.init(sh, q, pool + (size_t)unit * sh.K * AW::REC, b, h);
  // This wave's slots, 64 at a time; within a group two register buffers
  // alternate: while one block is processed the next one's loads are in flight.
  const int ns = a.n_slots(sh);
  for (int cb = 0; cb < ns; cb += kWave) {
    const int nv_l = a.slot_tokens(sh, p2l, unit, L, cb, ns);
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
    if (sa >= 0) a.load(a.slot_of(cb + sa), ka, va);
    while (sa >= 0) {
      const int sb = pop();
      if (sb >= 0) a.load(a.slot_of(cb + sb), kb, vb);
      a.process(ka, va, __builtin_amdgcn_readlane(nv_l, sa), scale_log2);
      if (sb < 0) break;
      sa = pop();
      if (sa >= 0) a.load(a.slot_of(cb + sa), ka, va);
      a.process(kb, vb, __builtin_amdgcn_readlane(nv_l, sb), scale_log2);
    }
  }
  a.merge_store(sh, b, h, out, lds);
}

// fp32 look-ahead attention: one wave per query row, 64 tokens (4 slots) per
// step, online softmax in fp32.
// LDS floats the fp32 path needs: per wave one query row and 64 weights.
__host__ __device__ constexpr int attn_f32_lds_bytes(int D) { return kWaves * (D + kWave) * 4; }

// fp32 path: one wave per stacked row; per group of four slots (64 tokens,
// one per lane) every key row and value column of the group is loaded at once
// (the loads do not wait on each other), the row's query and the 64 weights
// are broadcast through LDS, and the online softmax runs over the group.
// `lds`: attn_f32_lds_bytes(D) bytes.
template <int D>
__device__ __forceinline__ void attn_unit_f32(const Shape& sh, const float* __restrict__ q,
                                              const float* __restrict__ pool,
                                              const int32_t* __restrict__ p2l, int b, int h,
                                              int L, float scale, float* __restrict__ out,
                                              float* lds) {
  constexpr int REC = 2 * kBlock * D;
  constexpr int CPL = D / kWave;          // output channels per lane
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid % kWave;
  const int G = sh.G;
  const int K = sh.K;
  const int unit = b * sh.H + h;
  const float* unit_pool = pool + (size_t)unit * K * REC;
  float* qs = lds + w * (D + kWave);      // this wave's query row
  float* ps = qs + D;                     // the group's 64 weights
  const int32_t* slots = p2l + (size_t)unit * K;
  for (int r = w; r < 2 * G; r += kWaves) {
    const int row = r < G ? 0 : 1;
    const int head = h * G + (r < G ? r : r - G);
    const float* qr = q + ((size_t)(b * 2 + row) * sh.Hq + head) * D;
#pragma unroll
    for (int i = 0; i < CPL; ++i) qs[lane + kWave * i] = qr[lane + kWave * i];
    float m = -INFINITY, lsum = 0.f;
    float acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.f;
    for (int sb = 0; sb < K; sb += 4) {
      // lane = token u of slot sb + lane / 16
      const int s = sb + lane / kBlock;
      const int u = lane % kBlock;
      const int sc = s < K ? s : K - 1;                 // clamped, masked below
      const int j = slots[sc];
      const bool valid = s < K && j >= 0 && j < sh.NBmax && j * kBlock + u < L;
      const f32x4* kr = reinterpret_cast<const f32x4*>(unit_pool + (size_t)sc * REC + u * D);
      f32x4 kv[D / 4];
#pragma unroll
      for (int i = 0; i < D / 4; ++i) kv[i] = kr[i];
      // value columns of the group's four slots for this lane's channels
      f32x4 vv[CPL][4][4];
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int sq = sb + qq < K ? sb + qq : K - 1;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const f32x4* vc = reinterpret_cast<const f32x4*>(
              unit_pool + (size_t)sq * REC + kBlock * D + (lane + kWave * i) * kBlock);
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[i][qq][e] = vc[e];
        }
      }
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < D / 4; ++i) {
        const f32x4 q4 = reinterpret_cast<const f32x4*>(qs)[i];
        dot = fmaf(q4[0], kv[i][0], dot);
        dot = fmaf(q4[1], kv[i][1], dot);
        dot = fmaf(q4[2], kv[i][2], dot);
        dot = fmaf(q4[3], kv[i][3], dot);
      }
      const float z = valid ? dot * scale : -INFINITY;
      const float cm = wave_max(z);
      if (cm == -INFINITY) continue;                     // uniform across the wave
      const float nm = fmaxf(m, cm);
      const float f = (m == -INFINITY) ? 0.f : expf(m - nm);
      m = nm;
      lsum *= f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) acc[i] *= f;
      const float p = valid ? expf(z - m) : 0.f;
      lsum += wave_sum(p);
      ps[lane] = p;
      // values of tokens outside the resident set or the context never enter
      // the sum (whatever the pool holds there)
      const uint64_t vmask = ballot(valid);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x4 p4 = reinterpret_cast<const f32x4*>(ps)[4 * qq + e];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const bool in = (vmask >> (16 * qq + 4 * e + k)) & 1ull;
#pragma unroll
            for (int i = 0; i < CPL; ++i) acc[i] = fmaf(p4[k], in ? vv[i][qq][e][k] : 0.f, acc[i]);
          }
        }
      }
    }
    float* orow = out + ((size_t)(b * 2 + row) * sh.Hq + head) * D;
#pragma unroll
    for (int i = 0; i < CPL; ++i) orow[lane + kWave * i] = lsum > 0.f ? acc[i] / lsum : 0.f;
  }
}

}  // namespace oasis
