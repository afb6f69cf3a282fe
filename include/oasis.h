/*
 * oasis.h — C-ABI of the MI355X (gfx950) look-ahead sparse decode step.
 *
 * The method (OasisKV, "Scaling In-Decode KV Cache Beyond HBM with Lookahead
 * Sparse Prefetching", as described on the pith.science paper page, section
 * "What carries the argument", and the agihunt.info summary): for every
 * attention layer one attention pass runs the normal query and the
 * speculative draft query over the same per-KV-head resident set of sparse KV
 * blocks; the draft query then scans per-block min/max key summaries to rank
 * every logical block per KV head; a top-K selection and a capped eviction
 * (least-recently-selected victims) decide which blocks to stage in HBM for
 * the next step; the admitted blocks are copied from a host pool on a side
 * stream.
 *
 * ------------------------------------------------------------------------
 * Conventions shared by every call
 *
 *  Shape.  B requests, Hq query heads, Hkv KV heads (G = Hq / Hkv query heads
 *  per KV head, 1 <= G <= 16), head dim d in {64, 128}, block size S = 16
 *  tokens, NBmax logical blocks per (request, KV head) in the record and
 *  summary arrays (1 <= NBmax <= 8192), K resident slots per (request, KV
 *  head) (1 <= K <= 256), at most 2^22 units (B * Hkv).  Request b has
 *  ctx_len[b] valid tokens; its logical blocks are
 *  j < NB_b = min(ceil(ctx_len[b] / 16), NBmax).  A "unit" is one
 *  (request, KV head) pair, numbered b * Hkv + h.
 *
 *  Element type.  OASIS_DTYPE_F32 or OASIS_DTYPE_BF16 for queries, records,
 *  summaries and outputs (one type per shape).  Arithmetic is fp32.
 *
 *  Layouts (row-major, innermost last; all arrays contiguous):
 *   record     one logical block of one unit: keys [S][d] then values
 *              transposed [d][S]; 2*S*d elements.
 *   records    [B][Hkv][NBmax][record]  full KV (host pool or device)
 *   pool       [B][Hkv][K][record]      resident slots in HBM
 *   summ       [B][Hkv][NBmax][2][d]    [0] = min, [1] = max of the keys
 *   q, out     [B][2][Hq][d]            row 0 = normal, row 1 = draft query
 *   ctx_len    [B] int32
 *   l2p        [B][Hkv][NBmax] int32    slot holding logical block j, or -1
 *   p2l        [B][Hkv][K] int32        logical block held by slot s, or -1
 *   last_sel   [B][Hkv][K] int32        step the slot's block was last selected
 *   topk_idx   [B][Hkv][K] int32, topk_score [B][Hkv][K] float
 *   admit      [B][Hkv][K][3] int32     (logical, slot, evicted logical or -1)
 *   admit_count[B][Hkv] int32
 *
 *  Ownership.  Every buffer belongs to the caller; device pointers are HIP
 *  device (or host-mapped) addresses on the current device.  The library keeps
 *  no state between calls except a thread-local error string and the
 *  per-device scratch of oasis_layer_step_noalloc (a device array in the
 *  library's code object, not an allocation).  No call allocates device
 *  memory.
 *
 *  Asynchrony.  Each call enqueues its work on the given HIP stream (a
 *  hipStream_t passed as void*, NULL = the null stream) and returns without
 *  waiting, except oasis_prefetch in OASIS_PREFETCH_MEMCPY mode, which waits
 *  on the host for the admit list.
 *
 *  Errors.  Calls return OASIS_OK, or OASIS_ERR_INVALID (null pointer,
 *  inconsistent shape), OASIS_ERR_UNSUPPORTED (a size or type this build does
 *  not handle) before anything is enqueued, or OASIS_ERR_HIP when the HIP
 *  runtime reports an error.  oasis_last_error() returns a message for the
 *  calling thread's last failure.  No C++ exception crosses the ABI.  Device
 *  arrays are not inspected on the host: indices read from them are
 *  bounds-checked on the device and out-of-range entries are ignored.
 */
#ifndef OASIS_H
#define OASIS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum oasis_status {
    OASIS_OK = 0,
    OASIS_ERR_INVALID = 1,
    OASIS_ERR_UNSUPPORTED = 2,
    OASIS_ERR_HIP = 3
} oasis_status;

typedef enum oasis_dtype {
    OASIS_DTYPE_F32 = 0,
    OASIS_DTYPE_BF16 = 1
} oasis_dtype;

typedef enum oasis_prefetch_mode {
    OASIS_PREFETCH_GATHER = 0,  /* device gather kernel reading host-mapped memory */
    OASIS_PREFETCH_MEMCPY = 1   /* host waits for the admit list, then DMA copies */
} oasis_prefetch_mode;

typedef struct oasis_shape {
    int32_t batch;       /* B */
    int32_t n_q_heads;   /* Hq */
    int32_t n_kv_heads;  /* Hkv */
    int32_t head_dim;    /* d */
    int32_t block_size;  /* S, must be 16 */
    int32_t max_blocks;  /* NBmax */
    int32_t k_resident;  /* K */
    int32_t dtype;       /* oasis_dtype */
} oasis_shape;

/* Version of this ABI (incremented on any signature change). */
int32_t oasis_abi_version(void);

/* Message describing the calling thread's last failed call ("" if none). */
const char* oasis_last_error(void);

/* Admissions allowed per unit and step for a fetch ratio cap: floor(cap*K),
 * with a 1e-9 guard against binary rounding, clamped to [0, K].  The cap is
 * the per-step fetch ratio of the pith.science paper page's free parameters
 * (default 0.05) and of the agihunt.info fetch-cap ablation. */
int32_t oasis_cap_to_max_admit(double cap, int32_t k_resident);

/* Bytes of one block record, and of a whole summary array, of a shape. */
size_t oasis_record_bytes(const oasis_shape* shape);
size_t oasis_summary_bytes(const oasis_shape* shape);

/* Device address of pinned host memory (hipHostGetDevicePointer), for the
 * `records` argument of oasis_prefetch in gather mode and of oasis_summarize.
 * Returns OASIS_ERR_HIP if the memory is not pinned and mapped. */
oasis_status oasis_host_to_device_ptr(const void* host_ptr, void** device_ptr);

/* S0 — block summaries (pith.science paper page, "What carries the argument":
 * per-block coordinate-wise min/max of the keys, kept in HBM at about 1/16 of
 * the KV size).  For every unit and block j < NB_b writes summ[..][j][0][c] =
 * min and [1][c] = max of key channel c over the block's valid tokens; the
 * value written is one of the input values.  Entries j >= NB_b are not
 * written.  `records` may be device memory or host-mapped pinned memory. */
oasis_status oasis_summarize(const oasis_shape* shape, const void* records,
                             const int32_t* ctx_len, void* summ, void* stream);

/* S1 — look-ahead attention (pith.science paper page, "What carries the
 * argument": one kernel runs the normal and the draft token over the same
 * resident sparse KV set).  For both rows of every query head i (KV head
 * h = i / G): out = softmax(scale * q . k) v over the valid tokens (position
 * j*16 + u < ctx_len[b]) of the blocks j = p2l[s] >= 0 held by the unit's
 * slots, reading keys and values from pool slot s.  A unit with no valid
 * token gives 0.  `scale` <= 0 selects 1/sqrt(d). */
oasis_status oasis_lookahead_attn(const oasis_shape* shape, const void* q,
                                  const void* pool, const int32_t* p2l,
                                  const int32_t* ctx_len, float scale,
                                  void* out, void* stream);

/* S2+S3 — summary scan and top-K (pith.science paper page, "What carries the
 * argument": the draft query scans the summaries and ranks all logical blocks
 * per KV head; the pages' defaults are K = 128 blocks of 16 tokens).  Score of
 * block j < NB_b of unit (b, h):
 *     sum over the G query heads i of h, sum over channels c of
 *     max(q[b][q_row][i][c] * min[j][c], q[b][q_row][i][c] * max[j][c])
 * (unscaled; requires min <= max as oasis_summarize produces).  Writes the
 * min(K, NB_b) best blocks in the order (score descending, block ascending)
 * to topk_idx / topk_score (fp32 score); remaining entries get -1 / -inf.
 * q_row is 1 (draft) on the per-step path, 0 (normal) for a cold start.
 * When max_blocks exceeds 1024 the scan of a long context is split over one
 * workgroup per 1024-block part, whose lists go to `workspace` (device
 * memory, 256-byte aligned, at least oasis_layer_step_workspace_bytes(shape)
 * bytes; NULL allowed when that is 0); the last of a unit's parts to finish
 * merges them (one launch), and the result equals one scan over the whole
 * context.  The workspace needs no initialisation (its per-unit arrival
 * words carry a per-launch tag, so earlier contents count as zero); calls
 * that may run concurrently need separate workspaces. */
oasis_status oasis_score_topk(const oasis_shape* shape, const void* q,
                              int32_t q_row, const void* summ,
                              const int32_t* ctx_len, int32_t* topk_idx,
                              float* topk_score, void* workspace,
                              size_t workspace_bytes, void* stream);

/* S4 — capped eviction at step `step` (pith.science paper page, "What
 * carries the argument": admissions per step are capped and each admitted
 * non-resident block is paired with a least-recently-selected resident
 * block).  Per unit, in place on l2p / p2l / last_sel:
 *   1. slots whose block is in topk_idx get last_sel = step;
 *   2. M = blocks of topk_idx (in its order, -1 entries skipped) not resident;
 *   3. victims = empty slots in slot order, then slots with last_sel < step by
 *      (last_sel ascending, logical block ascending);
 *   4. a = min(max_admit, |M|, #victims); M[k] moves into victim k (k < a),
 *      the evicted block's l2p entry becomes -1, the slot is stamped `step`;
 *   5. admit[k] = (M[k], slot, evicted or -1) for k < a, -1 after;
 *      admit_count = a.
 * l2p and p2l must be mutual inverses on entry (they stay so). */
oasis_status oasis_capped_evict(const oasis_shape* shape,
                                const int32_t* topk_idx, int32_t step,
                                int32_t max_admit, int32_t* l2p, int32_t* p2l,
                                int32_t* last_sel, int32_t* admit,
                                int32_t* admit_count, void* stream);

/* S5 — prefetch (pith.science paper page, "What carries the argument": the
 * KV transfer stream; agihunt.info summary: decode is bound by the
 * host-to-GPU link).  Copies the whole record of every admitted block
 * (records[b][h][admit.logical]) into pool[b][h][admit.slot], for the first
 * admit_count[unit] entries of each unit (at most max_admit are read).
 * Enqueued on `side_stream` after waiting on `wait_before` (a hipEvent_t or
 * NULL); records `done` (a hipEvent_t or NULL) when the copies are enqueued.
 * GATHER mode: one kernel reads `records` through its device mapping
 * (host-mapped pinned memory or device memory); host_staging is unused.
 * MEMCPY mode: admit and admit_count are copied to `host_staging` (pinned
 * host memory of (B*Hkv*(3*K+1)) int32), the host waits for them, then the
 * records are copied with DMA (one hipMemcpyAsync per run of admissions
 * whose blocks and slots are both consecutive). */
oasis_status oasis_prefetch(const oasis_shape* shape, const void* records,
                            void* pool, const int32_t* admit,
                            const int32_t* admit_count, int32_t max_admit,
                            int32_t mode, int32_t* host_staging,
                            void* side_stream, void* wait_before, void* done);

/* Decode append (the step on either side of the layer step in a decode
 * loop).  The pith.science paper page ("What carries the argument") keeps the
 * full KV off HBM and the block summaries in HBM; the pages do not spell out
 * how a new token enters them, so this call takes the plain reading: the
 * token joins the block record that holds its position, the resident copy of
 * that block when it is resident, and that block's summary, and the context
 * grows by one.  For every request b with t = ctx_len[b] in [0, NBmax*16):
 * for every KV head h, k_new[b][h][:] becomes key row t%16 and v_new[b][h][:]
 * value column t%16 of records[b][h][t/16]; if pool is given and
 * l2p[b][h][t/16] = s is in [0, K), the same row and column are written into
 * pool slot s; summ[b][h][t/16] becomes (k, k) for the block's first token,
 * else its min/max widen to include k (a tie keeps the stored value); then
 * ctx_len[b] = t + 1.  Other requests are left unchanged.
 *   k_new, v_new  [B][Hkv][d] device memory, element type of the shape
 *   records       full KV, device or host-mapped pinned memory (written)
 *   pool, l2p     resident slots and slot map (device), both or neither NULL
 *   summ, ctx_len device memory (written)
 * Tokens earlier in the block must already be in records and summ. */
oasis_status oasis_append_token(const oasis_shape* shape, const void* k_new,
                                const void* v_new, void* records, void* pool,
                                const int32_t* l2p, void* summ,
                                int32_t* ctx_len, void* stream);

/* Top-K agreement diagnostic (a synthetic stand-in for the pith.science
 * paper page's "Core claim" measurement and the referee report on its
 * Fig. 6: the draft query's predicted top-K set against the exact top-K set
 * of the true next query).
 *
 * oasis_exact_topk: exact block scores from the keys, then the same top-K as
 * oasis_score_topk (same outputs, order and tie rule).  The exact score of
 * block j of unit (b, h) for query row q_row is the sum over the unit's G
 * query heads i of max over the block's valid tokens t of q_i . k_t
 * (unscaled): the quantity the summed Quest bounds of oasis_score_topk bound
 * from above.  `records` is the full KV [B][Hkv][NBmax][record] (device
 * memory; host-mapped memory works but reads over the host link).
 *
 * oasis_topk_agreement: per unit, counts[b][h][0] = entries among the first
 * exact_n (1 <= exact_n <= K) of exact_idx that lie in [0, NBmax), [1] = how
 * many of those pred_idx lists, [2] = how many of those are resident by l2p
 * (l2p[b][h][j] >= 0), or -1 when l2p is NULL.  exact_n = K compares whole
 * lists; a smaller exact_n asks for the recall of the exact list's best
 * blocks.  pred_idx, exact_idx [B][Hkv][K] int32 lists of distinct blocks
 * (-1 = unused); counts [B][Hkv][3] int32; all device memory. */
oasis_status oasis_exact_topk(const oasis_shape* shape, const void* q,
                              int32_t q_row, const void* records,
                              const int32_t* ctx_len, int32_t* topk_idx,
                              float* topk_score, void* stream);
oasis_status oasis_topk_agreement(const oasis_shape* shape,
                                  const int32_t* pred_idx,
                                  const int32_t* exact_idx,
                                  const int32_t* l2p, int32_t exact_n,
                                  int32_t* counts, void* stream);

/* Workspace bytes oasis_layer_step and oasis_score_topk need for a shape: 0
 * while max_blocks <= 1024, otherwise a few KiB per unit (the per-part top-K
 * lists of the split summary scan, the 1024 keys of a unit's last part, which
 * oasis_score_topk hands over unselected, and one 8-byte arrival word). */
size_t oasis_layer_step_workspace_bytes(const oasis_shape* shape);

/* S1..S4 fused — one look-ahead layer step in one launch: attention of both
 * rows over the current resident set (written to out), then the draft row's
 * summary scan, top-K and capped eviction as above.  Results are identical to
 * oasis_lookahead_attn, oasis_score_topk(q_row = 1) and oasis_capped_evict
 * called in that order on one stream.  When max_blocks exceeds 1024 the scan
 * of a long context is split over several workgroups whose partial top-K
 * lists go to `workspace` (device memory, 256-byte aligned, at least
 * oasis_layer_step_workspace_bytes(shape) bytes; NULL allowed when that is
 * 0); the last of the unit's workgroups to finish (the attention's
 * included) merges them and runs the eviction, all in one launch.  The
 * workspace needs no initialisation (as for oasis_score_topk); calls that may
 * run concurrently need separate workspaces. */
oasis_status oasis_layer_step(const oasis_shape* shape, const void* q,
                              const void* pool, const void* summ,
                              const int32_t* ctx_len, float scale,
                              int32_t step, int32_t max_admit, void* out,
                              int32_t* topk_idx, float* topk_score,
                              int32_t* l2p, int32_t* p2l, int32_t* last_sel,
                              int32_t* admit, int32_t* admit_count,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* The fused step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same launch and results as oasis_layer_step, with the split-scan
 * lists kept in the library's own device scratch instead of a workspace
 * argument.  The scratch is a 32 MiB array per device, held from the first
 * call on that device until the process ends; shapes whose lists exceed it
 * (oasis_layer_step_workspace_bytes above 32 MiB) return
 * OASIS_ERR_UNSUPPORTED.  The call allocates nothing.  All calls on one device
 * share its scratch: calls that may overlap on one device (other streams,
 * other threads) race and must be ordered by the caller.  The first call on a
 * device looks up the scratch's address (hipGetSymbolAddress); it is not
 * captured into a graph, so make one call before a capture begins. */
oasis_status oasis_layer_step_noalloc(const oasis_shape* shape, const void* q,
                                      const void* pool, const void* summ,
                                      const int32_t* ctx_len, float scale,
                                      int32_t step, int32_t max_admit, void* out,
                                      int32_t* topk_idx, float* topk_score,
                                      int32_t* l2p, int32_t* p2l,
                                      int32_t* last_sel, int32_t* admit,
                                      int32_t* admit_count, void* stream);

/* Dense comparator (not part of the look-ahead method) — decode attention of
 * both rows of every query head over every valid token of the full KV,
 * `records` [B][Hkv][NBmax][record] in device memory: the dense baseline the
 * pages compare against (agihunt.info summary, throughput table: dense vLLM).
 * Same output convention as oasis_lookahead_attn.  bf16 only.  `workspace`
 * (device memory, at least oasis_dense_attn_workspace_bytes(shape) bytes)
 * holds per-128-block partial results. */
size_t oasis_dense_attn_workspace_bytes(const oasis_shape* shape);
oasis_status oasis_dense_attn(const oasis_shape* shape, const void* q,
                              const void* records, const int32_t* ctx_len,
                              float scale, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* OASIS_H */
