// Host-only driver for the C-ABI layer (api.hip built as plain C++), run under
// AddressSanitizer and UBSan by tests/test_host_asan.py.  The HIP runtime
// calls the C-ABI layer makes are replaced by host stubs: copies are plain
// memcpy on host buffers, events and streams are no-ops.  The kernel
// launchers are replaced by stubs that count calls.  Exercised: argument
// validation of every entry point, the workspace checks of the fused step,
// and the MEMCPY prefetch mode end to end (staging of the admission list,
// planning of the copies as runs, the copies themselves) against a plain
// per-admission reference.
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "launch.h"
#include "oasis.h"

// ---------------------------------------------------------------- HIP stubs
static int g_memcpy_calls = 0;
static int g_fail_memcpy = 0;

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
  if (g_fail_memcpy) return hipErrorInvalidValue;
  ++g_memcpy_calls;
  memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned int) {
  *dev = host;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }

// ---------------------------------------------------------- launcher stubs
static int g_launches = 0;
static int g_last_gather_admit = -1;
static unsigned char g_scratch_stub[256] __attribute__((aligned(256)));
static int g_scratch_lookups = 0;

namespace oasis {
size_t layer_step_workspace_bytes(const Shape& sh) {
  return sh.NBmax > 1024 ? (size_t)sh.B * sh.H * 4096 : 0;
}
size_t dense_workspace_bytes(const Shape& sh) { return (size_t)sh.B * sh.H * 64; }
hipError_t scratch_pointer(void** ptr) {
  ++g_scratch_lookups;
  *ptr = g_scratch_stub;
  return hipSuccess;
}
hipError_t launch_summarize(const Shape&, int, const void*, const int32_t*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attn(const Shape&, int, const void*, const void*, const int32_t*, const int32_t*,
                       float, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_score_topk(const Shape&, int, const void*, int, const void*, const int32_t*,
                             int32_t*, float*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_exact_topk(const Shape&, int, const void*, int, const void*, const int32_t*,
                             int32_t*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_agreement(const Shape&, const int32_t*, const int32_t*, const int32_t*, int,
                            int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_evict(const Shape&, const int32_t*, int, int, int32_t*, int32_t*, int32_t*,
                        int32_t*, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_prefetch_gather(const Shape&, size_t, const void*, void*, const int32_t*,
                                  const int32_t*, int max_admit, hipStream_t) {
  ++g_launches;
  g_last_gather_admit = max_admit;
  return hipSuccess;
}
hipError_t launch_append(const Shape&, int, const void*, const void*, void*, void*, const int32_t*,
                         void*, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_layer_step(const Shape&, int, const void*, const void*, const void*,
                             const int32_t*, float, int, int, void*, int32_t*, float*, int32_t*,
                             int32_t*, int32_t*, int32_t*, int32_t*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_dense_attn(const Shape&, const void*, const void*, const int32_t*, float, void*,
                             void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace oasis

// ------------------------------------------------------------------ checks
static int g_failures = 0;
#define CHECK(cond)                                                         \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #cond);    \
      ++g_failures;                                                         \
    }                                                                       \
  } while (0)

static oasis_shape good_shape() {
  oasis_shape s = {4, 8, 2, 128, 16, 100, 16, OASIS_DTYPE_BF16};
  return s;
}

static void check_shape_validation() {
  char dummy[64];
  int32_t ctx[4] = {0, 0, 0, 0};
  struct Bad {
    oasis_shape s;
    oasis_status want;
  };
  oasis_shape g = good_shape();
  std::vector<Bad> bad;
  auto with = [&](void (*edit)(oasis_shape&), oasis_status want) {
    oasis_shape s = g;
    edit(s);
    bad.push_back({s, want});
  };
  with([](oasis_shape& s) { s.batch = -1; }, OASIS_ERR_INVALID);
  with([](oasis_shape& s) { s.n_kv_heads = 0; }, OASIS_ERR_INVALID);
  with([](oasis_shape& s) { s.n_q_heads = -8; }, OASIS_ERR_INVALID);
  with([](oasis_shape& s) { s.n_q_heads = 7; }, OASIS_ERR_INVALID);
  with([](oasis_shape& s) { s.n_q_heads = 34; }, OASIS_ERR_UNSUPPORTED);
  with([](oasis_shape& s) { s.head_dim = 96; }, OASIS_ERR_UNSUPPORTED);
  with([](oasis_shape& s) { s.block_size = 32; }, OASIS_ERR_UNSUPPORTED);
  with([](oasis_shape& s) { s.max_blocks = 0; }, OASIS_ERR_INVALID);
  with([](oasis_shape& s) { s.max_blocks = 8193; }, OASIS_ERR_UNSUPPORTED);
  with([](oasis_shape& s) { s.k_resident = 0; }, OASIS_ERR_INVALID);
  with([](oasis_shape& s) { s.k_resident = 257; }, OASIS_ERR_UNSUPPORTED);
  with([](oasis_shape& s) { s.dtype = 7; }, OASIS_ERR_UNSUPPORTED);
  with([](oasis_shape& s) { s.batch = 1 << 30; s.n_kv_heads = 8; s.n_q_heads = 8; },
       OASIS_ERR_UNSUPPORTED);
  const int before = g_launches;
  for (const Bad& b : bad) {
    CHECK(oasis_summarize(&b.s, dummy, ctx, dummy, nullptr) == b.want);
    CHECK(strlen(oasis_last_error()) > 0);
    CHECK(oasis_lookahead_attn(&b.s, dummy, dummy, ctx, ctx, 0.f, dummy, nullptr) == b.want);
    CHECK(oasis_score_topk(&b.s, dummy, 1, dummy, ctx, ctx, (float*)dummy, nullptr, 0, nullptr) ==
          b.want);
    CHECK(oasis_capped_evict(&b.s, ctx, 1, 1, ctx, ctx, ctx, ctx, ctx, nullptr) == b.want);
    CHECK(oasis_layer_step(&b.s, dummy, dummy, dummy, ctx, 0.f, 1, 1, dummy, ctx, (float*)dummy,
                           ctx, ctx, ctx, ctx, ctx, nullptr, 0, nullptr) == b.want);
  }
  CHECK(oasis_summarize(nullptr, dummy, ctx, dummy, nullptr) == OASIS_ERR_INVALID);
  CHECK(g_launches == before);
}

static void check_null_arguments() {
  oasis_shape s = good_shape();
  char d[64];
  int32_t c[4] = {0, 0, 0, 0};
  float* f = (float*)d;
  const int before = g_launches;
  CHECK(oasis_summarize(&s, nullptr, c, d, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_summarize(&s, d, nullptr, d, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_lookahead_attn(&s, d, d, nullptr, c, 0.f, d, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_lookahead_attn(&s, d, d, c, c, 1.f / 0.f, d, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_score_topk(&s, d, 2, d, c, c, f, nullptr, 0, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_score_topk(&s, d, 1, d, c, nullptr, f, nullptr, 0, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_capped_evict(&s, c, 1, -1, c, c, c, c, c, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_capped_evict(&s, c, 1, 1, c, c, nullptr, c, c, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_append_token(&s, d, d, d, d, nullptr, d, c, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_exact_topk(&s, d, 3, d, c, c, f, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_topk_agreement(&s, c, c, nullptr, 0, c, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_topk_agreement(&s, c, c, nullptr, s.k_resident + 1, c, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_prefetch(&s, d, d, c, c, 1, 5, nullptr, nullptr, nullptr, nullptr) ==
        OASIS_ERR_INVALID);
  CHECK(oasis_prefetch(&s, d, d, c, c, 1, OASIS_PREFETCH_MEMCPY, nullptr, nullptr, nullptr,
                       nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_dense_attn(&s, d, d, c, 0.f, d, nullptr, 0, nullptr) == OASIS_ERR_INVALID);
  oasis_shape f32 = s;
  f32.dtype = OASIS_DTYPE_F32;
  CHECK(oasis_dense_attn(&f32, d, d, c, 0.f, d, d, 1 << 20, nullptr) == OASIS_ERR_UNSUPPORTED);
  CHECK(oasis_host_to_device_ptr(nullptr, nullptr) == OASIS_ERR_INVALID);
  CHECK(g_launches == before);
  // batch 0: nothing to do, every pointer may be NULL
  oasis_shape z = s;
  z.batch = 0;
  CHECK(oasis_layer_step(&z, nullptr, nullptr, nullptr, nullptr, 0.f, 1, 6, nullptr, nullptr,
                         nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                         nullptr) == OASIS_OK);
  CHECK(g_launches == before);
}

static void check_layer_step_workspace() {
  oasis_shape s = good_shape();
  s.max_blocks = 3000;                            // split scan: a workspace is needed
  const size_t need = oasis_layer_step_workspace_bytes(&s);
  CHECK(need == (size_t)s.batch * s.n_kv_heads * 4096);
  std::vector<char> buf(need + 512);
  char* aligned = (char*)(((uintptr_t)buf.data() + 255) & ~(uintptr_t)255);
  char d[64];
  int32_t c[4] = {0, 0, 0, 0};
  float* f = (float*)d;
  const int before = g_launches;
  CHECK(oasis_layer_step(&s, d, d, d, c, 0.f, 1, 6, d, c, f, c, c, c, c, c, nullptr, need,
                         nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_layer_step(&s, d, d, d, c, 0.f, 1, 6, d, c, f, c, c, c, c, c, aligned, need - 1,
                         nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_layer_step(&s, d, d, d, c, 0.f, 1, 6, d, c, f, c, c, c, c, c, aligned + 4, need,
                         nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_layer_step(&s, d, d, d, c, 0.f, 1, -1, d, c, f, c, c, c, c, c, aligned, need,
                         nullptr) == OASIS_ERR_INVALID);
  CHECK(g_launches == before);
  CHECK(oasis_layer_step(&s, d, d, d, c, 0.f, 1, 6, d, c, f, c, c, c, c, c, aligned, need,
                         nullptr) == OASIS_OK);
  CHECK(g_launches == before + 1);
  // the standalone scan + top-K takes the same workspace
  CHECK(oasis_score_topk(&s, d, 1, d, c, c, f, nullptr, need, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_score_topk(&s, d, 1, d, c, c, f, aligned, need - 1, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_score_topk(&s, d, 1, d, c, c, f, aligned + 16, need, nullptr) == OASIS_ERR_INVALID);
  CHECK(oasis_score_topk(&s, d, 1, d, c, c, f, aligned, need, nullptr) == OASIS_OK);
  s.max_blocks = 1024;                            // one scan part: no workspace
  CHECK(oasis_layer_step_workspace_bytes(&s) == 0);
  CHECK(oasis_score_topk(&s, d, 1, d, c, c, f, nullptr, 0, nullptr) == OASIS_OK);
  CHECK(oasis_layer_step(&s, d, d, d, c, 0.f, 1, 6, d, c, f, c, c, c, c, c, nullptr, 0, nullptr) ==
        OASIS_OK);
}

static void check_layer_step_noalloc() {
  oasis_shape s = good_shape();
  char d[64];
  int32_t c[4] = {0, 0, 0, 0};
  float* f = (float*)d;
  const int before = g_launches, looked = g_scratch_lookups;
  // fits one scan part: no scratch needed
  CHECK(oasis_layer_step_noalloc(&s, d, d, d, c, 0.f, 1, 6, d, c, f, c, c, c, c, c, nullptr) ==
        OASIS_OK);
  CHECK(g_scratch_lookups == looked);
  // split scan within the scratch
  s.max_blocks = 3000;
  CHECK(oasis_layer_step_noalloc(&s, d, d, d, c, 0.f, 1, 6, d, c, f, c, c, c, c, c, nullptr) ==
        OASIS_OK);
  CHECK(g_scratch_lookups == looked + 1);
  CHECK(g_launches == before + 2);
  CHECK(oasis_layer_step_noalloc(&s, d, d, d, c, 0.f, 1, 6, nullptr, c, f, c, c, c, c, c,
                                 nullptr) == OASIS_ERR_INVALID);
  CHECK(strstr(oasis_last_error(), "oasis_layer_step_noalloc") != nullptr);
  // lists larger than the scratch are refused before anything is launched
  s.batch = (int)(oasis::kScratchBytes / 4096 / s.n_kv_heads) + 1;
  CHECK(oasis_layer_step_workspace_bytes(&s) > oasis::kScratchBytes);
  CHECK(oasis_layer_step_noalloc(&s, d, d, d, c, 0.f, 1, 6, d, c, f, c, c, c, c, c, nullptr) ==
        OASIS_ERR_UNSUPPORTED);
  CHECK(g_launches == before + 2);
}

static void check_helpers() {
  CHECK(oasis_cap_to_max_admit(0.05, 128) == 6);
  CHECK(oasis_cap_to_max_admit(0.25, 8) == 2);
  CHECK(oasis_cap_to_max_admit(0.01, 128) == 1);
  CHECK(oasis_cap_to_max_admit(1.0, 128) == 128);
  CHECK(oasis_cap_to_max_admit(3.0, 16) == 16);
  CHECK(oasis_cap_to_max_admit(0.0, 16) == 0);
  CHECK(oasis_cap_to_max_admit(-1.0, 16) == 0);
  CHECK(oasis_cap_to_max_admit(0.5, 0) == 0);
  oasis_shape s = good_shape();
  CHECK(oasis_record_bytes(&s) == 2 * 16 * 128 * 2);
  CHECK(oasis_summary_bytes(&s) == (size_t)4 * 2 * 100 * 2 * 128 * 2);
  CHECK(oasis_record_bytes(nullptr) == 0);
}

// MEMCPY prefetch: random admission lists (runs of consecutive blocks and
// slots, entries out of range, counts above max_admit) against a plain copy
// of every valid admission.
static void check_memcpy_prefetch(unsigned seed) {
  std::mt19937 rng(seed);
  oasis_shape s = good_shape();
  s.dtype = (seed & 1) ? OASIS_DTYPE_F32 : OASIS_DTYPE_BF16;
  s.head_dim = (seed & 2) ? 64 : 128;
  s.batch = 1 + (int)(rng() % 4);
  s.max_blocks = 1 + (int)(rng() % 60);
  s.k_resident = 1 + (int)(rng() % 20);
  const int units = s.batch * s.n_kv_heads, K = s.k_resident, NB = s.max_blocks;
  const size_t rec = oasis_record_bytes(&s);
  std::vector<unsigned char> records((size_t)units * NB * rec);
  for (auto& x : records) x = (unsigned char)rng();
  std::vector<unsigned char> pool((size_t)units * K * rec, 0xAB), want;
  std::vector<int32_t> admit((size_t)units * K * 3, -1), count(units, 0);
  const int max_admit = (int)(rng() % (K + 3));      // may exceed K: clamped
  for (int u = 0; u < units; ++u) {
    int n = (int)(rng() % (K + 1));
    int j = (int)(rng() % NB), sl = (int)(rng() % K);
    for (int k = 0; k < n; ++k) {
      if (rng() % 3 == 0) {                            // start a new run
        j = (int)(rng() % NB);
        sl = (int)(rng() % K);
      }
      int jj = j, ss = sl;
      if (rng() % 11 == 0) jj = (rng() & 1) ? -1 - (int)(rng() % 3) : NB + (int)(rng() % 3);
      if (rng() % 13 == 0) ss = (rng() & 1) ? -1 : K + (int)(rng() % 2);
      int32_t* a = &admit[((size_t)u * K + k) * 3];
      a[0] = jj;
      a[1] = ss;
      a[2] = -1;
      j = (j + 1) % NB;
      sl = (sl + 1) % K;
    }
    count[u] = n + ((rng() % 5 == 0) ? (int)(rng() % 4) : 0);   // may overstate the list
    if (count[u] > K) count[u] = K;
  }
  want = pool;
  const int m = max_admit < K ? max_admit : K;
  for (int u = 0; u < units; ++u) {
    int cnt = count[u] < m ? count[u] : m;
    for (int k = 0; k < cnt; ++k) {
      const int32_t* a = &admit[((size_t)u * K + k) * 3];
      if (a[0] < 0 || a[0] >= NB || a[1] < 0 || a[1] >= K) continue;
      memcpy(&want[((size_t)u * K + a[1]) * rec], &records[((size_t)u * NB + a[0]) * rec], rec);
    }
  }
  // the staging buffer has exactly the size the contract states
  int32_t* staging = (int32_t*)malloc(sizeof(int32_t) * (size_t)units * (3 * K + 1));
  g_memcpy_calls = 0;
  CHECK(oasis_prefetch(&s, records.data(), pool.data(), admit.data(), count.data(), max_admit,
                       OASIS_PREFETCH_MEMCPY, staging, nullptr, nullptr, nullptr) == OASIS_OK);
  free(staging);
  CHECK(pool == want);
  CHECK(max_admit == 0 || g_memcpy_calls >= 2);     // admission list and counts staged
  // gather mode hands the clamped quota to the kernel
  CHECK(oasis_prefetch(&s, records.data(), pool.data(), admit.data(), count.data(), max_admit,
                       OASIS_PREFETCH_GATHER, nullptr, nullptr, nullptr, nullptr) == OASIS_OK);
  CHECK(max_admit == 0 || g_last_gather_admit == m);
}

static void check_memcpy_runs_merge() {
  // one unit, blocks 3..7 into slots 0..4 and block 10 into slot 9: two copies
  // of records after the two staging copies
  oasis_shape s = {1, 2, 1, 64, 16, 16, 12, OASIS_DTYPE_F32};
  const size_t rec = oasis_record_bytes(&s);
  std::vector<unsigned char> records(16 * rec), pool(12 * rec, 0);
  for (size_t i = 0; i < records.size(); ++i) records[i] = (unsigned char)(i * 7 + 1);
  std::vector<int32_t> admit(12 * 3, -1), count(1, 6);
  const int jj[6] = {3, 4, 5, 6, 7, 10}, ss[6] = {0, 1, 2, 3, 4, 9};
  for (int k = 0; k < 6; ++k) {
    admit[k * 3] = jj[k];
    admit[k * 3 + 1] = ss[k];
  }
  std::vector<int32_t> staging(1 * (3 * 12 + 1));
  g_memcpy_calls = 0;
  CHECK(oasis_prefetch(&s, records.data(), pool.data(), admit.data(), count.data(), 6,
                       OASIS_PREFETCH_MEMCPY, staging.data(), nullptr, nullptr, nullptr) == OASIS_OK);
  CHECK(g_memcpy_calls == 2 + 2);
  for (int k = 0; k < 6; ++k)
    CHECK(memcmp(&pool[ss[k] * rec], &records[jj[k] * rec], rec) == 0);
  // a failing copy is reported, not hidden
  g_fail_memcpy = 1;
  CHECK(oasis_prefetch(&s, records.data(), pool.data(), admit.data(), count.data(), 6,
                       OASIS_PREFETCH_MEMCPY, staging.data(), nullptr, nullptr, nullptr) ==
        OASIS_ERR_HIP);
  g_fail_memcpy = 0;
  CHECK(strstr(oasis_last_error(), "oasis_prefetch") != nullptr);
}

int main() {
  check_shape_validation();
  check_null_arguments();
  check_layer_step_workspace();
  check_layer_step_noalloc();
  check_helpers();
  for (unsigned seed = 0; seed < 200; ++seed) check_memcpy_prefetch(seed);
  check_memcpy_runs_merge();
  if (g_failures) {
    fprintf(stderr, "%d host checks failed\n", g_failures);
    return 1;
  }
  printf("all host checks passed\n");
  return 0;
}
