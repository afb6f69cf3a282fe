// Exact block scores of the top-K agreement diagnostic (pith.science paper
// page, "Core claim" and the referee report on Fig. 6: the draft's predicted
// top-K set is compared with the exact top-K set of the true next query).
// The exact score of block j for KV head h is the sum over its G query heads
// of the largest logit q_i . k_t over the block's valid tokens: the quantity
// the summed Quest bounds of the scan bound from above.  The keys are read
// from the full KV, so the scan streams half of every record of the unit.
#pragma once

#include "common.h"

namespace oasis {

// Max over the 16 lanes of a DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return x;
}

// bf16: one wave per block, U blocks in flight per wave.  The logit tile is
// D[token][head] = K[token][:] . Q[head][:] (mfma 16x16x32 bf16, D/32 steps),
// so lane (g, n) holds head n, tokens 4g..4g+3; heads n >= G have a zero
// query and are left out of the sum.  Writes keys[j] = score_key(score).
template <int D, int U>
__device__ __forceinline__ void exact_scan_bf16(const Shape& sh, const uint16_t* __restrict__ q,
                                                int q_row, const uint16_t* __restrict__ rec_unit,
                                                int b, int h, int L, int nb, uint32_t* keys) {
  constexpr int KS = D / 32;
  constexpr int REC = 2 * kBlock * D;
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  const int g = lane >> 4, n = lane & 15;
  const bool head = n < sh.G;
  bf16x8 qop[KS];
  const uint16_t* qr = q + ((size_t)(b * 2 + q_row) * sh.Hq + h * sh.G + (head ? n : 0)) * D;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    if (head) {
      qop[kk] = *reinterpret_cast<const bf16x8*>(qr + 32 * kk + 8 * g);
    } else {
      u32x4 z = {0u, 0u, 0u, 0u};
      qop[kk] = __builtin_bit_cast(bf16x8, z);
    }
  }
  for (int j0 = w * U; j0 < nb; j0 += kWaves * U) {
    bf16x8 kr[U][KS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u < nb ? j0 + u : nb - 1;   // in-range duplicate, not used
      const uint16_t* rec = rec_unit + (size_t)j * REC + n * D + 8 * g;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        kr[u][kk] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(rec + 32 * kk));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u;
      if (j >= nb) break;                             // uniform over the wave
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[u][kk], qop[kk], z, 0, 0, 0);
      const int nv = L - j * kBlock;
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * g + i < nv) m = fmaxf(m, z[i]);
      m = xrow_max(m);
      const float s = row16_sum(head ? m : 0.f);
      if (lane == 0) keys[j] = score_key(s);
    }
  }
}

// fp32: VALU, one wave per block; lane (g, n) takes token n and channels
// g*D/4 .. +D/4, the four channel quarters are summed across lanes and the
// token max is taken over the 16 lanes of a row, head by head.
template <int D>
__device__ __forceinline__ void exact_scan_f32(const Shape& sh, const float* __restrict__ q,
                                               int q_row, const float* __restrict__ rec_unit,
                                               int b, int h, int L, int nb, uint32_t* keys) {
  constexpr int CPL = D / 4;
  constexpr int REC = 2 * kBlock * D;
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  const int g = lane >> 4, n = lane & 15;
  const int c0 = g * CPL;
  for (int j = w; j < nb; j += kWaves) {
    float k[CPL];
    const float* rec = rec_unit + (size_t)j * REC + n * D + c0;
#pragma unroll
    for (int c = 0; c < CPL; c += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(rec + c);
      k[c] = v[0]; k[c + 1] = v[1]; k[c + 2] = v[2]; k[c + 3] = v[3];
    }
    const bool valid = n < L - j * kBlock;
    float s = 0.f;
    for (int i = 0; i < sh.G; ++i) {
      const float* qi = q + ((size_t)(b * 2 + q_row) * sh.Hq + h * sh.G + i) * D + c0;
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) part = fmaf(qi[c], k[c], part);
      const float dot = xrow_sum(part);
      s += row16_max(valid ? dot : -INFINITY);
    }
    if (lane == 0) keys[j] = score_key(s);
  }
}

}  // namespace oasis
