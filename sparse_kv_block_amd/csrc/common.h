// Device helpers shared by the gfx950 kernels: element loads, bf16 packing,
// wave64 reductions and orderable score keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace oasis {

constexpr int kWave = 64;
constexpr int kBlock = 16;      // tokens per KV block
constexpr int kThreads = 256;   // threads per workgroup (4 waves) in every per-unit kernel
constexpr int kWaves = kThreads / kWave;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int n_blocks(int L, int NBmax) {
  if (L <= 0) return 0;
  const int nb = L / kBlock + (L % kBlock != 0);     // no overflow near INT_MAX
  return nb < NBmax ? nb : NBmax;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// DPP lane moves inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Integer DPP move; lanes whose source is outside the row (or whose row is
// not in ROWS) get 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts inside each
// 16-lane row, then the row totals broadcast into the rows above.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += dpp_i<0x111>(x);        // row_shr:1
  x += dpp_i<0x112>(x);        // row_shr:2
  x += dpp_i<0x114>(x);        // row_shr:4
  x += dpp_i<0x118>(x);        // row_shr:8
  x += dpp_i<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_i<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// Bitwise OR over the 64 lanes of a wave (a wave-uniform value).
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
  x |= (uint32_t)dpp_i<0xB1>((int)x);    // quad_perm [1,0,3,2]
  x |= (uint32_t)dpp_i<0x4E>((int)x);    // quad_perm [2,3,0,1]
  x |= (uint32_t)dpp_i<0x141>((int)x);   // row_half_mirror
  x |= (uint32_t)dpp_i<0x140>((int)x);   // row_mirror
  return (uint32_t)(__builtin_amdgcn_readlane((int)x, 0) | __builtin_amdgcn_readlane((int)x, 16) |
                    __builtin_amdgcn_readlane((int)x, 32) | __builtin_amdgcn_readlane((int)x, 48));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}

// Max / sum over lanes l, l^16, l^32, l^48 (the four lanes that share l % 16).
// Lane l's value beside that of lane l ^ 16 (l ^ 32): v_permlane16_swap
// (v_permlane32_swap) on two copies of x leaves the two values of every lane
// pair in (a, b) in both lanes, as VALU moves with no LDS round trip.
__device__ __forceinline__ void xor16_pair(float x, float& a, float& b) {
  const u32x2 r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void xor32_pair(float x, float& a, float& b) {
  const u32x2 r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                   false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// Reductions over lanes l, l ^ 16, l ^ 32, l ^ 48 (the same lane of the four
// 16-lane rows); min, max and the two-operand sums are commutative, so the
// result is the same in all four lanes.
__device__ __forceinline__ float xrow_max(float x) {
  float a, b;
  xor16_pair(x, a, b);
  xor32_pair(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xrow_min(float x) {
  float a, b;
  xor16_pair(x, a, b);
  xor32_pair(fminf(a, b), a, b);
  return fminf(a, b);
}
__device__ __forceinline__ float xrow_sum(float x) {
  float a, b;
  xor16_pair(x, a, b);
  xor32_pair(a + b, a, b);
  return a + b;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0 and +0
// map to the same key.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int lane_id() { return __lane_id(); }
// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---- split summary scan of long contexts ----
constexpr int kScanChunk = 1024;   // blocks per scan part

struct StepWorkspace {
  uint32_t* key;                 // [units][parts][K]  a scan part's list, padded with key 0
  int32_t* idx;                  // [units][parts][K]
  uint32_t* raw;                 // [units][kScanChunk]  the last scan part's keys, unselected
  unsigned long long* arrive;    // [units]  tagged arrival count of the fused step
  unsigned long long tag;        // this launch's tag (bits 16..63, odd there; bits 0..15 zero)
};

// Scan parts of a context (at least one), and the workgroup slots per unit of
// a fused-step launch: one when every context fits one scan part; otherwise
// one for the attention plus one per scan part of the longest context.
__host__ __device__ inline int scan_parts(int nb) {
  return nb > kScanChunk ? (nb + kScanChunk - 1) / kScanChunk : 1;
}
__host__ __device__ inline int step_parts(int NBmax) {
  return NBmax > kScanChunk ? 1 + scan_parts(NBmax) : 1;
}

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline size_t step_workspace_bytes(int units, int parts, int K) {
  if (parts <= 1) return 0;
  return 2 * align256((size_t)units * parts * K * 4) + align256((size_t)units * kScanChunk * 4) +
         align256((size_t)units * 8);
}

__host__ __device__ inline StepWorkspace step_workspace(void* base, int units, int parts, int K) {
  StepWorkspace w{nullptr, nullptr, nullptr, nullptr, 0};
  if (parts <= 1 || base == nullptr) return w;
  char* p = static_cast<char*>(base);
  w.key = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)units * parts * K * 4);
  w.idx = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)units * parts * K * 4);
  w.raw = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)units * kScanChunk * 4);
  w.arrive = reinterpret_cast<unsigned long long*>(p);
  return w;
}

}  // namespace oasis
