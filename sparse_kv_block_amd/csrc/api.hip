// C-ABI of liboasis: argument validation, error reporting and dispatch to the
// gfx950 launchers.  Declarations and contracts: include/oasis.h.  Host code
// only (HIP runtime API and the launchers of launch.h), so that it also builds
// as plain C++ for the sanitizer test of its validation and copy planning.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "launch.h"
#include "oasis.h"

namespace {

thread_local std::string g_error;

oasis_status fail(oasis_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

oasis_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return OASIS_OK;
  return fail(OASIS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

using oasis::kMaxBlocks;
constexpr int kMaxK = 256;
constexpr int kMaxGroup = 16;
// Units per call: keeps every per-launch count the kernels form in 32-bit
// ints (units x 256 slots, units x 9 scan parts, units x 64 dense chunks).
constexpr int kMaxUnits = 1 << 22;

oasis_status check_shape(const oasis_shape* s, const char* fn) {
  if (!s) return fail(OASIS_ERR_INVALID, "%s: shape is NULL", fn);
  if (s->batch < 0) return fail(OASIS_ERR_INVALID, "%s: batch %d < 0", fn, s->batch);
  if (s->n_kv_heads <= 0 || s->n_q_heads <= 0)
    return fail(OASIS_ERR_INVALID, "%s: head counts must be positive (Hq %d, Hkv %d)", fn,
                s->n_q_heads, s->n_kv_heads);
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(OASIS_ERR_INVALID, "%s: Hq %d is not a multiple of Hkv %d", fn, s->n_q_heads,
                s->n_kv_heads);
  if (s->n_q_heads / s->n_kv_heads > kMaxGroup)
    return fail(OASIS_ERR_UNSUPPORTED, "%s: %d query heads per KV head (at most %d)", fn,
                s->n_q_heads / s->n_kv_heads, kMaxGroup);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(OASIS_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, s->head_dim);
  if (s->block_size != 16)
    return fail(OASIS_ERR_UNSUPPORTED, "%s: block_size %d (must be 16)", fn, s->block_size);
  if (s->max_blocks <= 0) return fail(OASIS_ERR_INVALID, "%s: max_blocks %d", fn, s->max_blocks);
  if (s->max_blocks > kMaxBlocks)
    return fail(OASIS_ERR_UNSUPPORTED, "%s: max_blocks %d (at most %d)", fn, s->max_blocks,
                kMaxBlocks);
  if (s->k_resident <= 0) return fail(OASIS_ERR_INVALID, "%s: k_resident %d", fn, s->k_resident);
  if (s->k_resident > kMaxK)
    return fail(OASIS_ERR_UNSUPPORTED, "%s: k_resident %d (at most %d)", fn, s->k_resident, kMaxK);
  if (s->dtype != OASIS_DTYPE_F32 && s->dtype != OASIS_DTYPE_BF16)
    return fail(OASIS_ERR_UNSUPPORTED, "%s: dtype %d", fn, s->dtype);
  if ((long long)s->batch * s->n_kv_heads > kMaxUnits)
    return fail(OASIS_ERR_UNSUPPORTED, "%s: %lld units (batch x KV heads, at most %d)", fn,
                (long long)s->batch * s->n_kv_heads, kMaxUnits);
  return OASIS_OK;
}

oasis::Shape to_shape(const oasis_shape* s) {
  oasis::Shape sh;
  sh.B = s->batch;
  sh.Hq = s->n_q_heads;
  sh.H = s->n_kv_heads;
  sh.G = s->n_q_heads / s->n_kv_heads;
  sh.d = s->head_dim;
  sh.NBmax = s->max_blocks;
  sh.K = s->k_resident;
  return sh;
}

size_t esize(const oasis_shape* s) { return s->dtype == OASIS_DTYPE_F32 ? 4 : 2; }

#define OASIS_NONNULL(ptr, fn)                                                  \
  do {                                                                          \
    if (!(ptr)) return fail(OASIS_ERR_INVALID, "%s: %s is NULL", fn, #ptr);     \
  } while (0)

// The split-scan workspace of oasis_score_topk and oasis_layer_step: none
// while every context fits one scan part, else at least the bytes
// oasis_layer_step_workspace_bytes gives, 256-byte aligned.
oasis_status check_workspace(const oasis_shape* shape, const void* workspace,
                             size_t workspace_bytes, const char* fn) {
  const size_t need = oasis::layer_step_workspace_bytes(to_shape(shape));
  if (need == 0) return OASIS_OK;
  if (!workspace) return fail(OASIS_ERR_INVALID, "%s: workspace is NULL (%zu bytes needed)", fn, need);
  if (workspace_bytes < need)
    return fail(OASIS_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                need);
  if (((uintptr_t)workspace & 255) != 0)
    return fail(OASIS_ERR_INVALID, "%s: workspace must be 256-byte aligned", fn);
  return OASIS_OK;
}

}  // namespace

extern "C" {

int32_t oasis_abi_version(void) { return 8; }

const char* oasis_last_error(void) { return g_error.c_str(); }

int32_t oasis_cap_to_max_admit(double cap, int32_t k) {
  if (!(cap > 0.0) || k <= 0) return 0;
  double m = floor(cap * (double)k + 1e-9);
  if (m > k) m = k;
  return (int32_t)m;
}

size_t oasis_record_bytes(const oasis_shape* s) {
  if (!s) return 0;
  return (size_t)2 * s->block_size * s->head_dim * esize(s);
}

size_t oasis_summary_bytes(const oasis_shape* s) {
  if (!s) return 0;
  return (size_t)s->batch * s->n_kv_heads * s->max_blocks * 2 * s->head_dim * esize(s);
}

oasis_status oasis_host_to_device_ptr(const void* host_ptr, void** device_ptr) {
  const char* fn = "oasis_host_to_device_ptr";
  OASIS_NONNULL(host_ptr, fn);
  OASIS_NONNULL(device_ptr, fn);
  return hip_status(hipHostGetDevicePointer(device_ptr, const_cast<void*>(host_ptr), 0), fn);
}

oasis_status oasis_summarize(const oasis_shape* shape, const void* records, const int32_t* ctx_len,
                             void* summ, void* stream) {
  const char* fn = "oasis_summarize";
  if (oasis_status st = check_shape(shape, fn)) return st;
  if (shape->batch == 0) return OASIS_OK;
  OASIS_NONNULL(records, fn);
  OASIS_NONNULL(ctx_len, fn);
  OASIS_NONNULL(summ, fn);
  return hip_status(oasis::launch_summarize(to_shape(shape), shape->dtype, records, ctx_len, summ,
                                            (hipStream_t)stream),
                    fn);
}

oasis_status oasis_lookahead_attn(const oasis_shape* shape, const void* q, const void* pool,
                                  const int32_t* p2l, const int32_t* ctx_len, float scale, void* out,
                                  void* stream) {
  const char* fn = "oasis_lookahead_attn";
  if (oasis_status st = check_shape(shape, fn)) return st;
  if (shape->batch == 0) return OASIS_OK;
  OASIS_NONNULL(q, fn);
  OASIS_NONNULL(pool, fn);
  OASIS_NONNULL(p2l, fn);
  OASIS_NONNULL(ctx_len, fn);
  OASIS_NONNULL(out, fn);
  if (isnan(scale) || isinf(scale)) return fail(OASIS_ERR_INVALID, "%s: scale is not finite", fn);
  return hip_status(oasis::launch_attn(to_shape(shape), shape->dtype, q, pool, p2l, ctx_len, scale,
                                       out, (hipStream_t)stream),
                    fn);
}

oasis_status oasis_score_topk(const oasis_shape* shape, const void* q, int32_t q_row,
                              const void* summ, const int32_t* ctx_len, int32_t* topk_idx,
                              float* topk_score, void* workspace, size_t workspace_bytes,
                              void* stream) {
  const char* fn = "oasis_score_topk";
  if (oasis_status st = check_shape(shape, fn)) return st;
  if (q_row != 0 && q_row != 1) return fail(OASIS_ERR_INVALID, "%s: q_row %d (0 or 1)", fn, q_row);
  if (shape->batch == 0) return OASIS_OK;
  OASIS_NONNULL(q, fn);
  OASIS_NONNULL(summ, fn);
  OASIS_NONNULL(ctx_len, fn);
  OASIS_NONNULL(topk_idx, fn);
  OASIS_NONNULL(topk_score, fn);
  if (oasis_status st = check_workspace(shape, workspace, workspace_bytes, fn)) return st;
  return hip_status(oasis::launch_score_topk(to_shape(shape), shape->dtype, q, q_row, summ, ctx_len,
                                             topk_idx, topk_score, workspace, (hipStream_t)stream),
                    fn);
}

oasis_status oasis_capped_evict(const oasis_shape* shape, const int32_t* topk_idx, int32_t step,
                                int32_t max_admit, int32_t* l2p, int32_t* p2l, int32_t* last_sel,
                                int32_t* admit, int32_t* admit_count, void* stream) {
  const char* fn = "oasis_capped_evict";
  if (oasis_status st = check_shape(shape, fn)) return st;
  if (max_admit < 0) return fail(OASIS_ERR_INVALID, "%s: max_admit %d < 0", fn, max_admit);
  if (shape->batch == 0) return OASIS_OK;
  OASIS_NONNULL(topk_idx, fn);
  OASIS_NONNULL(l2p, fn);
  OASIS_NONNULL(p2l, fn);
  OASIS_NONNULL(last_sel, fn);
  OASIS_NONNULL(admit, fn);
  OASIS_NONNULL(admit_count, fn);
  return hip_status(oasis::launch_evict(to_shape(shape), topk_idx, step, max_admit, l2p, p2l,
                                        last_sel, admit, admit_count, (hipStream_t)stream),
                    fn);
}

oasis_status oasis_prefetch(const oasis_shape* shape, const void* records, void* pool,
                            const int32_t* admit, const int32_t* admit_count, int32_t max_admit,
                            int32_t mode, int32_t* host_staging, void* side_stream,
                            void* wait_before, void* done) {
  const char* fn = "oasis_prefetch";
  if (oasis_status st = check_shape(shape, fn)) return st;
  if (max_admit < 0) return fail(OASIS_ERR_INVALID, "%s: max_admit %d < 0", fn, max_admit);
  if (mode != OASIS_PREFETCH_GATHER && mode != OASIS_PREFETCH_MEMCPY)
    return fail(OASIS_ERR_INVALID, "%s: mode %d", fn, mode);
  OASIS_NONNULL(records, fn);
  OASIS_NONNULL(pool, fn);
  OASIS_NONNULL(admit, fn);
  OASIS_NONNULL(admit_count, fn);
  if (mode == OASIS_PREFETCH_MEMCPY) OASIS_NONNULL(host_staging, fn);
  if (max_admit > shape->k_resident) max_admit = shape->k_resident;
  hipStream_t st = (hipStream_t)side_stream;
  if (wait_before) {
    if (oasis_status s = hip_status(hipStreamWaitEvent(st, (hipEvent_t)wait_before, 0), fn)) return s;
  }
  const oasis::Shape sh = to_shape(shape);
  const size_t rec_bytes = oasis_record_bytes(shape);
  if (shape->batch > 0 && max_admit > 0) {
    if (mode == OASIS_PREFETCH_GATHER) {
      if (oasis_status s = hip_status(oasis::launch_prefetch_gather(sh, rec_bytes, records, pool, admit,
                                                                    admit_count, max_admit, st),
                                      fn))
        return s;
    } else {
      const size_t units = (size_t)sh.B * sh.H;
      const size_t admit_elems = units * sh.K * 3;
      if (oasis_status s = hip_status(hipMemcpyAsync(host_staging, admit, admit_elems * 4,
                                                     hipMemcpyDefault, st), fn)) return s;
      if (oasis_status s = hip_status(hipMemcpyAsync(host_staging + admit_elems, admit_count,
                                                     units * 4, hipMemcpyDefault, st), fn)) return s;
      if (oasis_status s = hip_status(hipStreamSynchronize(st), fn)) return s;
      // One DMA copy per run of admissions whose logical blocks and slots are
      // both consecutive (a run is one contiguous range on each side).
      const char* src_base = (const char*)records;
      char* dst_base = (char*)pool;
      for (size_t u = 0; u < units; ++u) {
        int cnt = host_staging[admit_elems + u];
        if (cnt > max_admit) cnt = max_admit;
        int run_j = -1, run_s = -1, run_n = 0;
        for (int k = 0; k <= cnt; ++k) {
          int j = -1, s = -1;
          if (k < cnt) {
            const int32_t* a = host_staging + (u * sh.K + k) * 3;
            j = a[0];
            s = a[1];
            if (j < 0 || j >= sh.NBmax || s < 0 || s >= sh.K) j = s = -1;
          }
          if (run_n > 0 && j == run_j + run_n && s == run_s + run_n) {
            ++run_n;
            continue;
          }
          if (run_n > 0) {
            hipError_t e = hipMemcpyAsync(dst_base + (u * sh.K + run_s) * rec_bytes,
                                          src_base + (u * sh.NBmax + run_j) * rec_bytes,
                                          run_n * rec_bytes, hipMemcpyDefault, st);
            if (oasis_status r = hip_status(e, fn)) return r;
          }
          run_j = j;
          run_s = s;
          run_n = j >= 0 ? 1 : 0;
        }
      }
    }
  }
  if (done) {
    if (oasis_status s = hip_status(hipEventRecord((hipEvent_t)done, st), fn)) return s;
  }
  return OASIS_OK;
}

oasis_status oasis_append_token(const oasis_shape* shape, const void* k_new, const void* v_new,
                                void* records, void* pool, const int32_t* l2p, void* summ,
                                int32_t* ctx_len, void* stream) {
  const char* fn = "oasis_append_token";
  if (oasis_status st = check_shape(shape, fn)) return st;
  if (shape->batch == 0) return OASIS_OK;
  OASIS_NONNULL(k_new, fn);
  OASIS_NONNULL(v_new, fn);
  OASIS_NONNULL(records, fn);
  OASIS_NONNULL(summ, fn);
  OASIS_NONNULL(ctx_len, fn);
  if ((pool == nullptr) != (l2p == nullptr))
    return fail(OASIS_ERR_INVALID, "%s: pool and l2p must both be given or both be NULL", fn);
  return hip_status(oasis::launch_append(to_shape(shape), shape->dtype, k_new, v_new, records, pool,
                                         l2p, summ, ctx_len, (hipStream_t)stream),
                    fn);
}

oasis_status oasis_exact_topk(const oasis_shape* shape, const void* q, int32_t q_row,
                              const void* records, const int32_t* ctx_len, int32_t* topk_idx,
                              float* topk_score, void* stream) {
  const char* fn = "oasis_exact_topk";
  if (oasis_status st = check_shape(shape, fn)) return st;
  if (q_row != 0 && q_row != 1) return fail(OASIS_ERR_INVALID, "%s: q_row %d (0 or 1)", fn, q_row);
  if (shape->batch == 0) return OASIS_OK;
  OASIS_NONNULL(q, fn);
  OASIS_NONNULL(records, fn);
  OASIS_NONNULL(ctx_len, fn);
  OASIS_NONNULL(topk_idx, fn);
  OASIS_NONNULL(topk_score, fn);
  return hip_status(oasis::launch_exact_topk(to_shape(shape), shape->dtype, q, q_row, records,
                                             ctx_len, topk_idx, topk_score, (hipStream_t)stream),
                    fn);
}

oasis_status oasis_topk_agreement(const oasis_shape* shape, const int32_t* pred_idx,
                                  const int32_t* exact_idx, const int32_t* l2p, int32_t exact_n,
                                  int32_t* counts, void* stream) {
  const char* fn = "oasis_topk_agreement";
  if (oasis_status st = check_shape(shape, fn)) return st;
  if (exact_n <= 0 || exact_n > shape->k_resident)
    return fail(OASIS_ERR_INVALID, "%s: exact_n %d (1 .. K = %d)", fn, exact_n, shape->k_resident);
  if (shape->batch == 0) return OASIS_OK;
  OASIS_NONNULL(pred_idx, fn);
  OASIS_NONNULL(exact_idx, fn);
  OASIS_NONNULL(counts, fn);
  return hip_status(oasis::launch_agreement(to_shape(shape), pred_idx, exact_idx, l2p, exact_n,
                                            counts, (hipStream_t)stream),
                    fn);
}

size_t oasis_layer_step_workspace_bytes(const oasis_shape* shape) {
  if (!shape || shape->n_kv_heads <= 0 || shape->batch <= 0 || shape->max_blocks <= 0 ||
      shape->k_resident <= 0)
    return 0;
  return oasis::layer_step_workspace_bytes(to_shape(shape));
}

}  // extern "C"

namespace {

// Validation and launch shared by oasis_layer_step (caller's workspace) and
// oasis_layer_step_noalloc (the library's scratch, `use_scratch`).
oasis_status layer_step_impl(const char* fn, bool use_scratch, const oasis_shape* shape,
                             const void* q, const void* pool, const void* summ,
                             const int32_t* ctx_len, float scale, int32_t step, int32_t max_admit,
                             void* out, int32_t* topk_idx, float* topk_score, int32_t* l2p,
                             int32_t* p2l, int32_t* last_sel, int32_t* admit, int32_t* admit_count,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (oasis_status st = check_shape(shape, fn)) return st;
  if (max_admit < 0) return fail(OASIS_ERR_INVALID, "%s: max_admit %d < 0", fn, max_admit);
  if (isnan(scale) || isinf(scale)) return fail(OASIS_ERR_INVALID, "%s: scale is not finite", fn);
  const size_t need = oasis_layer_step_workspace_bytes(shape);
  if (use_scratch && need > oasis::kScratchBytes)
    return fail(OASIS_ERR_UNSUPPORTED,
                "%s: this shape needs %zu bytes of split-scan lists, above the library's "
                "%zu-byte scratch (oasis_layer_step takes a workspace of any size)",
                fn, need, oasis::kScratchBytes);
  if (shape->batch == 0) return OASIS_OK;
  OASIS_NONNULL(q, fn);
  OASIS_NONNULL(pool, fn);
  OASIS_NONNULL(summ, fn);
  OASIS_NONNULL(ctx_len, fn);
  OASIS_NONNULL(out, fn);
  OASIS_NONNULL(topk_idx, fn);
  OASIS_NONNULL(topk_score, fn);
  OASIS_NONNULL(l2p, fn);
  OASIS_NONNULL(p2l, fn);
  OASIS_NONNULL(last_sel, fn);
  OASIS_NONNULL(admit, fn);
  OASIS_NONNULL(admit_count, fn);
  if (need > 0 && use_scratch) {
    if (oasis_status s = hip_status(oasis::scratch_pointer(&workspace), fn)) return s;
  } else if (oasis_status st = check_workspace(shape, workspace, workspace_bytes, fn)) {
    return st;
  }
  return hip_status(oasis::launch_layer_step(to_shape(shape), shape->dtype, q, pool, summ, ctx_len,
                                             scale, step, max_admit, out, topk_idx, topk_score, l2p,
                                             p2l, last_sel, admit, admit_count,
                                             need > 0 ? workspace : nullptr, (hipStream_t)stream),
                    fn);
}

}  // namespace

extern "C" {

oasis_status oasis_layer_step(const oasis_shape* shape, const void* q, const void* pool,
                              const void* summ, const int32_t* ctx_len, float scale, int32_t step,
                              int32_t max_admit, void* out, int32_t* topk_idx, float* topk_score,
                              int32_t* l2p, int32_t* p2l, int32_t* last_sel, int32_t* admit,
                              int32_t* admit_count, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return layer_step_impl("oasis_layer_step", false, shape, q, pool, summ, ctx_len, scale, step,
                         max_admit, out, topk_idx, topk_score, l2p, p2l, last_sel, admit,
                         admit_count, workspace, workspace_bytes, stream);
}

oasis_status oasis_layer_step_noalloc(const oasis_shape* shape, const void* q, const void* pool,
                                      const void* summ, const int32_t* ctx_len, float scale,
                                      int32_t step, int32_t max_admit, void* out,
                                      int32_t* topk_idx, float* topk_score, int32_t* l2p,
                                      int32_t* p2l, int32_t* last_sel, int32_t* admit,
                                      int32_t* admit_count, void* stream) {
  return layer_step_impl("oasis_layer_step_noalloc", true, shape, q, pool, summ, ctx_len, scale,
                         step, max_admit, out, topk_idx, topk_score, l2p, p2l, last_sel, admit,
                         admit_count, nullptr, 0, stream);
}

size_t oasis_dense_attn_workspace_bytes(const oasis_shape* shape) {
  if (check_shape(shape, "oasis_dense_attn_workspace_bytes") != OASIS_OK) return 0;
  return oasis::dense_workspace_bytes(to_shape(shape));
}

oasis_status oasis_dense_attn(const oasis_shape* shape, const void* q, const void* records,
                              const int32_t* ctx_len, float scale, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const char* fn = "oasis_dense_attn";
  if (oasis_status st = check_shape(shape, fn)) return st;
  if (shape->dtype != OASIS_DTYPE_BF16)
    return fail(OASIS_ERR_UNSUPPORTED, "%s: bf16 only", fn);
  if (isnan(scale) || isinf(scale)) return fail(OASIS_ERR_INVALID, "%s: scale is not finite", fn);
  if (shape->batch == 0) return OASIS_OK;
  OASIS_NONNULL(q, fn);
  OASIS_NONNULL(records, fn);
  OASIS_NONNULL(ctx_len, fn);
  OASIS_NONNULL(out, fn);
  OASIS_NONNULL(workspace, fn);
  const size_t need = oasis::dense_workspace_bytes(to_shape(shape));
  if (workspace_bytes < need)
    return fail(OASIS_ERR_INVALID, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes, need);
  return hip_status(oasis::launch_dense_attn(to_shape(shape), q, records, ctx_len, scale, out,
                                             workspace, (hipStream_t)stream),
                    fn);
}

}  // extern "C"
