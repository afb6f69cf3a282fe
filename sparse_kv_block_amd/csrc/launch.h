// Internal launchers: the kernels' translation unit exports these to the
// C-ABI layer.  Arguments are already validated by the caller.  Host code
// only: the C-ABI layer includes nothing else from the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace oasis {

// Validated problem shape: B requests, Hq query heads, H KV heads, G = Hq / H,
// head dim d, NBmax blocks per unit in the record and summary arrays, K slots.
struct Shape {
  int B, Hq, H, G, d, NBmax, K;
};

// Most blocks per unit (NBmax) the kernels accept.
constexpr int kMaxBlocks = 8192;

// Bytes of the fused step's split-scan workspace for a shape (0 when every
// context fits one scan part).
size_t layer_step_workspace_bytes(const Shape& sh);

// The library's own device scratch (oasis_layer_step_noalloc): its size, and
// its address on the current device (looked up on the first call per device).
constexpr size_t kScratchBytes = (size_t)32 << 20;
hipError_t scratch_pointer(void** ptr);

hipError_t launch_summarize(const Shape& sh, int dtype, const void* records,
                            const int32_t* ctx_len, void* summ, hipStream_t st);
hipError_t launch_attn(const Shape& sh, int dtype, const void* q, const void* pool,
                       const int32_t* p2l, const int32_t* ctx_len, float scale, void* out,
                       hipStream_t st);
hipError_t launch_score_topk(const Shape& sh, int dtype, const void* q, int q_row,
                             const void* summ, const int32_t* ctx_len, int32_t* topk_idx,
                             float* topk_score, void* workspace, hipStream_t st);
hipError_t launch_exact_topk(const Shape& sh, int dtype, const void* q, int q_row,
                             const void* records, const int32_t* ctx_len, int32_t* topk_idx,
                             float* topk_score, hipStream_t st);
hipError_t launch_agreement(const Shape& sh, const int32_t* pred, const int32_t* exact,
                            const int32_t* l2p, int exact_n, int32_t* counts, hipStream_t st);
hipError_t launch_evict(const Shape& sh, const int32_t* topk_idx, int step, int max_admit,
                        int32_t* l2p, int32_t* p2l, int32_t* last_sel, int32_t* admit,
                        int32_t* admit_count, hipStream_t st);
hipError_t launch_prefetch_gather(const Shape& sh, size_t rec_bytes, const void* records,
                                  void* pool, const int32_t* admit, const int32_t* admit_count,
                                  int max_admit, hipStream_t st);
hipError_t launch_append(const Shape& sh, int dtype, const void* k_new, const void* v_new,
                         void* records, void* pool, const int32_t* l2p, void* summ,
                         int32_t* ctx_len, hipStream_t st);
hipError_t launch_layer_step(const Shape& sh, int dtype, const void* q, const void* pool,
                             const void* summ, const int32_t* ctx_len, float scale, int step,
                             int max_admit, void* out, int32_t* topk_idx, float* topk_score,
                             int32_t* l2p, int32_t* p2l, int32_t* last_sel, int32_t* admit,
                             int32_t* admit_count, void* workspace, hipStream_t st);

size_t dense_workspace_bytes(const Shape& sh);
hipError_t launch_dense_attn(const Shape& sh, const void* q, const void* records,
                             const int32_t* ctx_len, float scale, void* out, void* workspace,
                             hipStream_t st);

}  // namespace oasis
