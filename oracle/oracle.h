/*
 * Plain fp64 CPU oracle of the OasisKV look-ahead sparse decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the HIP library and includes nothing from it.
 *
 * Sources (the OasisKV pages):
 *  - pith.science paper page, "What carries the argument": one attention pass
 *    runs the normal and the draft token over the same resident sparse KV set;
 *    the draft query scans per-block coordinate-wise min/max key summaries
 *    (Quest style) and ranks every logical block per KV head; a capped
 *    eviction pairs each admitted non-resident block with a
 *    least-recently-selected resident block.
 *  - pith.science paper page, "Assumptions & free parameters": block size 16,
 *    K = 128 blocks, fetch cap 0.05, summaries about 1/16 of the KV size.
 *  - agihunt.info summary, fetch-cap ablation paragraph: per-step traffic is
 *    bounded by the cap.
 *
 * Element types: dtype 0 = IEEE float32, dtype 1 = bfloat16 (raw 16-bit
 * patterns).  All arithmetic is double precision.
 *
 * Array layouts (row-major, innermost last):
 *   records  [B][H][NBmax][2*S*d]: keys [S][d] then transposed values [d][S]
 *   summ     [B][H][NBmax][2][d]: [0] = coordinate-wise min, [1] = max
 *   q, out   [B][2][Hq][d]: row 0 = normal query, row 1 = draft query
 *   l2p      [B][H][NBmax] int32: slot holding the logical block, or -1
 *   p2l      [B][H][K] int32: logical block held by the slot, or -1
 *   last_sel [B][H][K] int32: step at which the slot's block was last selected
 *   admit    [B][H][K][3] int32: (logical, slot, evicted logical or -1)
 *
 * A "unit" is one (request b, KV head h) pair, numbered b*H + h.  Every
 * function takes an optional list of units (NULL = all) and touches only the
 * outputs of the listed units.  nthreads <= 1 runs on the calling thread.
 */
#ifndef OASIS_ORACLE_H
#define OASIS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

void ora_summarize(int B, int H, int NBmax, int S, int d, int dtype,
                   const void* records, const int32_t* ctx_len, void* summ,
                   const int32_t* units, int n_units, int nthreads);

void ora_block_scores(int B, int Hq, int H, int NBmax, int S, int d, int dtype,
                      const void* q, int q_row, const void* summ,
                      const int32_t* ctx_len, double* scores,
                      const int32_t* units, int n_units, int nthreads);

/* Exact block scores (ground truth of the top-K agreement diagnostic): per
 * block, the sum over the G query heads of the largest logit q_i . k_t over
 * the block's valid tokens (keys read from `records`). */
void ora_exact_block_scores(int B, int Hq, int H, int NBmax, int S, int d, int dtype,
                            const void* q, int q_row, const void* records,
                            const int32_t* ctx_len, double* scores,
                            const int32_t* units, int n_units, int nthreads);

void ora_topk(int B, int H, int NBmax, int S, int K, const double* scores,
              const int32_t* ctx_len, int32_t* topk_idx, double* topk_score,
              const int32_t* units, int n_units);

int  ora_max_admit(double cap, int K);

void ora_capped_evict(int B, int H, int NBmax, int K, const int32_t* topk_idx,
                      int32_t step, int32_t max_admit, int32_t* l2p,
                      int32_t* p2l, int32_t* last_sel, int32_t* admit,
                      int32_t* admit_count, const int32_t* units, int n_units);

void ora_attention(int B, int Hq, int H, int NBmax, int S, int d, int K,
                   int dtype, const void* q, const void* records,
                   const int32_t* p2l, const int32_t* ctx_len, double scale,
                   double* out, const int32_t* units, int n_units, int nthreads);

void ora_prefetch(int B, int H, int NBmax, int S, int d, int K, int dtype,
                  const void* records, void* pool, const int32_t* admit,
                  const int32_t* admit_count, const int32_t* units, int n_units);

/* Decode append: request b's new token (position t = ctx_len[b]) goes into
 * key row t%S and value column t%S of block t/S of records (and of pool slot
 * l2p[block] when that block is resident; pool may be NULL); the block's
 * summary becomes min/max over its tokens 0..t%S; ctx_len[b] grows by one.
 * Requests whose next position is past NBmax*S are left unchanged.
 * k_new, v_new: [B][H][d]. */
void ora_append(int B, int H, int NBmax, int S, int d, int K, int dtype,
                const void* k_new, const void* v_new, void* records, void* pool,
                const int32_t* l2p, void* summ, int32_t* ctx_len);

#ifdef __cplusplus
}
#endif
#endif
