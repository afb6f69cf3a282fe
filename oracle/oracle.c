/*
 * Plain fp64 CPU oracle of the OasisKV look-ahead sparse decode step.
 * TEST INFRASTRUCTURE ONLY: see oracle.h for the contract, the layouts and the
 * page citations.  Written for reading, not for speed: no blocking, no fusion,
 * each step is the definition written out.
 */
#define _GNU_SOURCE
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* element access                                                            */

static double elem(const void* base, int dtype, size_t i) {
    if (dtype == 0) return (double)((const float*)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static size_t esize(int dtype) { return dtype == 0 ? 4 : 2; }

/* number of logical blocks of a request: ceil(L/S), never above NBmax */
static int n_blocks(int32_t L, int S, int NBmax) {
    if (L <= 0) return 0;
    int nb = (int)((L + S - 1) / S);
    return nb < NBmax ? nb : NBmax;
}

/* ------------------------------------------------------------------------ */
/* unit-parallel driver                                                      */

typedef void (*unit_fn)(void* ctx, int unit);

typedef struct {
    unit_fn fn;
    void* ctx;
    const int32_t* units;
    int n_units;
    int first, last;
} span_t;

static void* run_span(void* p) {
    span_t* s = (span_t*)p;
    for (int k = s->first; k < s->last; ++k)
        s->fn(s->ctx, s->units ? s->units[k] : k);
    return NULL;
}

static void for_units(unit_fn fn, void* ctx, const int32_t* units, int n_units,
                      int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n_units) nthreads = n_units > 0 ? n_units : 1;
    if (nthreads == 1) {
        span_t s = {fn, ctx, units, n_units, 0, n_units};
        run_span(&s);
        return;
    }
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    span_t* sp = (span_t*)malloc(sizeof(span_t) * (size_t)nthreads);
    for (int t = 0; t < nthreads; ++t) {
        sp[t].fn = fn; sp[t].ctx = ctx; sp[t].units = units; sp[t].n_units = n_units;
        sp[t].first = (int)((long long)n_units * t / nthreads);
        sp[t].last = (int)((long long)n_units * (t + 1) / nthreads);
        pthread_create(&th[t], NULL, run_span, &sp[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(sp);
}

/* ------------------------------------------------------------------------ */
/* Summaries: coordinate-wise min and max of the keys of each block
 * (pith.science paper page, "What carries the argument": per-block min/max key
 * summaries in the style of Quest).  Only the valid tokens of a partial last
 * block take part.  The result is one of the inputs, so it is copied bit for
 * bit; among equal values the first token wins.                              */

typedef struct {
    int H, NBmax, S, d, dtype;
    const void* rec;
    const int32_t* ctx_len;
    void* summ;
} summ_ctx;

static void summarize_unit(void* p, int unit) {
    summ_ctx* c = (summ_ctx*)p;
    int b = unit / c->H;
    int32_t L = c->ctx_len[b];
    int nb = n_blocks(L, c->S, c->NBmax);
    size_t es = esize(c->dtype);
    size_t rec_elems = (size_t)2 * c->S * c->d;
    for (int j = 0; j < nb; ++j) {
        size_t rbase = ((size_t)unit * c->NBmax + j) * rec_elems;
        size_t sbase = ((size_t)unit * c->NBmax + j) * 2 * (size_t)c->d;
        int nvalid = L - j * c->S;
        if (nvalid > c->S) nvalid = c->S;
        for (int ch = 0; ch < c->d; ++ch) {
            size_t imin = rbase + ch, imax = rbase + ch;      /* token 0 */
            double vmin = elem(c->rec, c->dtype, imin), vmax = vmin;
            for (int u = 1; u < nvalid; ++u) {
                size_t i = rbase + (size_t)u * c->d + ch;
                double v = elem(c->rec, c->dtype, i);
                if (v < vmin) { vmin = v; imin = i; }
                if (v > vmax) { vmax = v; imax = i; }
            }
            memcpy((char*)c->summ + (sbase + ch) * es, (const char*)c->rec + imin * es, es);
            memcpy((char*)c->summ + (sbase + c->d + ch) * es, (const char*)c->rec + imax * es, es);
        }
    }
}

void ora_summarize(int B, int H, int NBmax, int S, int d, int dtype,
                   const void* records, const int32_t* ctx_len, void* summ,
                   const int32_t* units, int n_units, int nthreads) {
    summ_ctx c = {H, NBmax, S, d, dtype, records, ctx_len, summ};
    for_units(summarize_unit, &c, units, units ? n_units : B * H, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Block scores: the draft query scans the summaries and scores every logical
 * block of the KV head (pith.science paper page, "What carries the argument").
 * Per query head the Quest bound is sum_c max(q_c*min_c, q_c*max_c); the G
 * query heads that share the KV head are summed.  Blocks past the context get
 * -inf.  Summation order: heads outer, channels inner.                      */

typedef struct {
    int Hq, H, NBmax, S, d, dtype, q_row;
    const void* q;
    const void* summ;
    const int32_t* ctx_len;
    double* scores;
} score_ctx;

static void score_unit(void* p, int unit) {
    score_ctx* c = (score_ctx*)p;
    int b = unit / c->H, h = unit % c->H;
    int G = c->Hq / c->H;
    int nb = n_blocks(c->ctx_len[b], c->S, c->NBmax);
    for (int j = 0; j < c->NBmax; ++j) {
        double s = -INFINITY;
        if (j < nb) {
            size_t sbase = ((size_t)unit * c->NBmax + j) * 2 * (size_t)c->d;
            s = 0.0;
            for (int i = h * G; i < (h + 1) * G; ++i) {
                size_t qbase = (((size_t)b * 2 + c->q_row) * c->Hq + i) * (size_t)c->d;
                for (int ch = 0; ch < c->d; ++ch) {
                    double qv = elem(c->q, c->dtype, qbase + ch);
                    double lo = elem(c->summ, c->dtype, sbase + ch);
                    double hi = elem(c->summ, c->dtype, sbase + c->d + ch);
                    double a = qv * lo, e = qv * hi;
                    s += (a > e) ? a : e;
                }
            }
        }
        c->scores[(size_t)unit * c->NBmax + j] = s;
    }
}

void ora_block_scores(int B, int Hq, int H, int NBmax, int S, int d, int dtype,
                      const void* q, int q_row, const void* summ,
                      const int32_t* ctx_len, double* scores,
                      const int32_t* units, int n_units, int nthreads) {
    score_ctx c = {Hq, H, NBmax, S, d, dtype, q_row, q, summ, ctx_len, scores};
    for_units(score_unit, &c, units, units ? n_units : B * H, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Exact block scores, the ground truth the draft's prediction is compared
 * with (pith.science paper page, "Core claim" and the referee report on
 * Fig. 6: the propagated draft query's top-K set against the exact top-K set
 * of the true next-token query).  Per query head the exact score of a block
 * is the largest logit q . k_t over its valid tokens t; the G query heads of
 * the KV head are summed, exactly as the Quest bounds are summed, so that the
 * bound is never below it.  Blocks past the context get -inf.              */

typedef struct {
    int Hq, H, NBmax, S, d, dtype, q_row;
    const void* q;
    const void* rec;
    const int32_t* ctx_len;
    double* scores;
} exact_ctx;

static void exact_unit(void* p, int unit) {
    exact_ctx* c = (exact_ctx*)p;
    int b = unit / c->H, h = unit % c->H;
    int G = c->Hq / c->H;
    int32_t L = c->ctx_len[b];
    int nb = n_blocks(L, c->S, c->NBmax);
    size_t rec_elems = (size_t)2 * c->S * c->d;
    for (int j = 0; j < c->NBmax; ++j) {
        double s = -INFINITY;
        if (j < nb) {
            size_t rbase = ((size_t)unit * c->NBmax + j) * rec_elems;
            int nvalid = L - j * c->S;
            if (nvalid > c->S) nvalid = c->S;
            s = 0.0;
            for (int i = h * G; i < (h + 1) * G; ++i) {
                size_t qbase = (((size_t)b * 2 + c->q_row) * c->Hq + i) * (size_t)c->d;
                double best = -INFINITY;
                for (int u = 0; u < nvalid; ++u) {
                    double logit = 0.0;
                    for (int ch = 0; ch < c->d; ++ch)
                        logit += elem(c->q, c->dtype, qbase + ch) *
                                 elem(c->rec, c->dtype, rbase + (size_t)u * c->d + ch);
                    if (logit > best) best = logit;
                }
                s += best;
            }
        }
        c->scores[(size_t)unit * c->NBmax + j] = s;
    }
}

void ora_exact_block_scores(int B, int Hq, int H, int NBmax, int S, int d, int dtype,
                            const void* q, int q_row, const void* records,
                            const int32_t* ctx_len, double* scores,
                            const int32_t* units, int n_units, int nthreads) {
    exact_ctx c = {Hq, H, NBmax, S, d, dtype, q_row, q, records, ctx_len, scores};
    for_units(exact_unit, &c, units, units ? n_units : B * H, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Top-K: the K best blocks of the unit by (score descending, block index
 * ascending), listed in that order; all blocks if the request has at most K.
 * Unused entries are index -1, score -inf.                                   */

typedef struct { double s; int32_t j; } scored_t;

static int by_score_then_index(const void* x, const void* y) {
    const scored_t* a = (const scored_t*)x;
    const scored_t* b = (const scored_t*)y;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->j < b->j) ? -1 : (a->j > b->j);
}

void ora_topk(int B, int H, int NBmax, int S, int K, const double* scores,
              const int32_t* ctx_len, int32_t* topk_idx, double* topk_score,
              const int32_t* units, int n_units) {
    int n = units ? n_units : B * H;
    scored_t* tmp = (scored_t*)malloc(sizeof(scored_t) * (size_t)(NBmax > 0 ? NBmax : 1));
    for (int k = 0; k < n; ++k) {
        int unit = units ? units[k] : k;
        int nb = n_blocks(ctx_len[unit / H], S, NBmax);
        for (int j = 0; j < nb; ++j) {
            tmp[j].s = scores[(size_t)unit * NBmax + j];
            tmp[j].j = j;
        }
        qsort(tmp, (size_t)nb, sizeof(scored_t), by_score_then_index);
        for (int r = 0; r < K; ++r) {
            topk_idx[(size_t)unit * K + r] = r < nb ? tmp[r].j : -1;
            if (topk_score) topk_score[(size_t)unit * K + r] = r < nb ? tmp[r].s : -INFINITY;
        }
    }
    free(tmp);
}

/* ------------------------------------------------------------------------ */
/* Admissions allowed per KV head and step: floor(cap*K).  The pages give the
 * cap as a fetch ratio (pith.science paper page, free parameters: 0.05); the
 * 1e-9 guard keeps products like 0.25*8 from rounding down to 1.            */

int ora_max_admit(double cap, int K) {
    if (!(cap > 0.0)) return 0;
    double m = floor(cap * (double)K + 1e-9);
    if (m > K) m = K;
    return (int)m;
}

/* ------------------------------------------------------------------------ */
/* Capped eviction at step t (pith.science paper page, "What carries the
 * argument": the cap bounds admissions per step and each admitted
 * non-resident block is paired with a least-recently-selected resident block).
 * Per unit:
 *   1. every resident block that is in T is stamped "selected at t";
 *   2. M = the members of T, in T's order, that are not resident;
 *   3. victims: empty slots in slot order, then resident slots whose stamp is
 *      older than t, by (stamp ascending, logical block ascending);
 *   4. a = min(max_admit, |M|, number of victims); the k-th admitted block
 *      M[k] replaces the k-th victim and is stamped t;
 *   5. admit[k] = (M[k], slot, evicted block or -1); unused entries are -1.  */

typedef struct { int32_t stamp, logical, slot; } victim_t;

static int by_stamp_then_logical(const void* x, const void* y) {
    const victim_t* a = (const victim_t*)x;
    const victim_t* b = (const victim_t*)y;
    if (a->stamp != b->stamp) return a->stamp < b->stamp ? -1 : 1;
    return (a->logical < b->logical) ? -1 : (a->logical > b->logical);
}

void ora_capped_evict(int B, int H, int NBmax, int K, const int32_t* topk_idx,
                      int32_t step, int32_t max_admit, int32_t* l2p,
                      int32_t* p2l, int32_t* last_sel, int32_t* admit,
                      int32_t* admit_count, const int32_t* units, int n_units) {
    int n = units ? n_units : B * H;
    int32_t* missing = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    victim_t* old = (victim_t*)malloc(sizeof(victim_t) * (size_t)K);
    for (int k = 0; k < n; ++k) {
        int unit = units ? units[k] : k;
        const int32_t* T = topk_idx + (size_t)unit * K;
        int32_t* L2P = l2p + (size_t)unit * NBmax;
        int32_t* P2L = p2l + (size_t)unit * K;
        int32_t* LS = last_sel + (size_t)unit * K;
        int32_t* AD = admit + (size_t)unit * K * 3;

        /* 1 and 2 */
        int nm = 0;
        for (int r = 0; r < K; ++r) {
            int32_t j = T[r];
            if (j < 0) continue;
            int32_t s = L2P[j];
            if (s >= 0) LS[s] = step;
            else missing[nm++] = j;
        }
        /* 3 */
        int nv = 0, no = 0;
        for (int s = 0; s < K; ++s)
            if (P2L[s] < 0) order[nv++] = s;
        for (int s = 0; s < K; ++s)
            if (P2L[s] >= 0 && LS[s] < step) {
                old[no].stamp = LS[s]; old[no].logical = P2L[s]; old[no].slot = s; ++no;
            }
        qsort(old, (size_t)no, sizeof(victim_t), by_stamp_then_logical);
        for (int r = 0; r < no; ++r) order[nv++] = old[r].slot;
        /* 4 */
        int a = max_admit < nm ? max_admit : nm;
        if (a > nv) a = nv;
        if (a < 0) a = 0;
        for (int r = 0; r < a; ++r) {
            int32_t s = order[r];
            int32_t ev = P2L[s];
            if (ev >= 0) L2P[ev] = -1;
            P2L[s] = missing[r];
            L2P[missing[r]] = s;
            LS[s] = step;
            AD[3 * r + 0] = missing[r];
            AD[3 * r + 1] = s;
            AD[3 * r + 2] = ev;
        }
        /* 5 */
        for (int r = a; r < K; ++r) AD[3 * r] = AD[3 * r + 1] = AD[3 * r + 2] = -1;
        admit_count[unit] = a;
    }
    free(missing);
    free(order);
    free(old);
}

/* ------------------------------------------------------------------------ */
/* Look-ahead attention (pith.science paper page, "What carries the argument":
 * one pass runs the normal and the draft token over the same resident sparse
 * set).  For every query row (normal and draft) of every query head i, with
 * KV head h = i / G: softmax(scale * q . k) over the valid tokens of the
 * blocks that the unit's slots hold, times v.  Keys and values are read from
 * the logical records, so a slot's pool copy is not consulted.  An empty set
 * gives 0.                                                                   */

typedef struct {
    int Hq, H, NBmax, S, d, K, dtype;
    const void* q;
    const void* rec;
    const int32_t* p2l;
    const int32_t* ctx_len;
    double scale;
    double* out;
} attn_ctx;

static void attention_unit(void* p, int unit) {
    attn_ctx* c = (attn_ctx*)p;
    int b = unit / c->H, h = unit % c->H;
    int G = c->Hq / c->H;
    int32_t L = c->ctx_len[b];
    size_t rec_elems = (size_t)2 * c->S * c->d;
    int maxtok = c->K * c->S;
    size_t* kbase = (size_t*)malloc(sizeof(size_t) * (size_t)(maxtok > 0 ? maxtok : 1));
    size_t* vbase = (size_t*)malloc(sizeof(size_t) * (size_t)(maxtok > 0 ? maxtok : 1));
    double* z = (double*)malloc(sizeof(double) * (size_t)(maxtok > 0 ? maxtok : 1));
    int nt = 0;
    for (int s = 0; s < c->K; ++s) {
        int32_t j = c->p2l[(size_t)unit * c->K + s];
        if (j < 0 || j >= c->NBmax) continue;
        for (int u = 0; u < c->S; ++u) {
            if ((long long)j * c->S + u >= L) continue;
            size_t r = ((size_t)unit * c->NBmax + j) * rec_elems;
            kbase[nt] = r + (size_t)u * c->d;                 /* key row u */
            vbase[nt] = r + (size_t)c->S * c->d + u;           /* value column u */
            ++nt;
        }
    }
    for (int row = 0; row < 2; ++row) {
        for (int i = h * G; i < (h + 1) * G; ++i) {
            size_t qb = (((size_t)b * 2 + row) * c->Hq + i) * (size_t)c->d;
            double* o = c->out + qb;
            for (int ch = 0; ch < c->d; ++ch) o[ch] = 0.0;
            if (nt == 0) continue;
            double zmax = -INFINITY;
            for (int t = 0; t < nt; ++t) {
                double acc = 0.0;
                for (int ch = 0; ch < c->d; ++ch)
                    acc += elem(c->q, c->dtype, qb + ch) * elem(c->rec, c->dtype, kbase[t] + ch);
                z[t] = c->scale * acc;
                if (z[t] > zmax) zmax = z[t];
            }
            double denom = 0.0;
            for (int t = 0; t < nt; ++t) { z[t] = exp(z[t] - zmax); denom += z[t]; }
            for (int t = 0; t < nt; ++t) {
                double w = z[t] / denom;
                for (int ch = 0; ch < c->d; ++ch)
                    o[ch] += w * elem(c->rec, c->dtype, vbase[t] + (size_t)ch * c->S);
            }
        }
    }
    free(kbase);
    free(vbase);
    free(z);
}

void ora_attention(int B, int Hq, int H, int NBmax, int S, int d, int K,
                   int dtype, const void* q, const void* records,
                   const int32_t* p2l, const int32_t* ctx_len, double scale,
                   double* out, const int32_t* units, int n_units, int nthreads) {
    attn_ctx c = {Hq, H, NBmax, S, d, K, dtype, q, records, p2l, ctx_len, scale, out};
    for_units(attention_unit, &c, units, units ? n_units : B * H, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Prefetch: every admitted block's whole record is copied into its slot.    */

void ora_prefetch(int B, int H, int NBmax, int S, int d, int K, int dtype,
                  const void* records, void* pool, const int32_t* admit,
                  const int32_t* admit_count, const int32_t* units, int n_units) {
    int n = units ? n_units : B * H;
    size_t rec_bytes = (size_t)2 * S * d * esize(dtype);
    for (int k = 0; k < n; ++k) {
        int unit = units ? units[k] : k;
        for (int r = 0; r < admit_count[unit]; ++r) {
            int32_t j = admit[((size_t)unit * K + r) * 3 + 0];
            int32_t s = admit[((size_t)unit * K + r) * 3 + 1];
            memcpy((char*)pool + ((size_t)unit * K + s) * rec_bytes,
                   (const char*)records + ((size_t)unit * NBmax + j) * rec_bytes, rec_bytes);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Decode append (the token the next step adds to the context).  The summary
 * of the tail block is recomputed from its stored keys, which is the plain
 * definition of the min/max over the block's valid tokens.                  */

void ora_append(int B, int H, int NBmax, int S, int d, int K, int dtype,
                const void* k_new, const void* v_new, void* records, void* pool,
                const int32_t* l2p, void* summ, int32_t* ctx_len) {
    size_t es = esize(dtype);
    size_t rec_elems = (size_t)2 * S * d;
    for (int b = 0; b < B; ++b) {
        int32_t t = ctx_len[b];
        if (t < 0 || t >= NBmax * S) continue;
        int j = t / S, u = t % S;
        for (int h = 0; h < H; ++h) {
            int unit = b * H + h;
            char* rec = (char*)records + ((size_t)unit * NBmax + j) * rec_elems * es;
            for (int c = 0; c < d; ++c) {
                memcpy(rec + ((size_t)u * d + c) * es,
                       (const char*)k_new + ((size_t)unit * d + c) * es, es);
                memcpy(rec + ((size_t)S * d + (size_t)c * S + u) * es,
                       (const char*)v_new + ((size_t)unit * d + c) * es, es);
            }
            if (pool) {
                int32_t s = l2p[(size_t)unit * NBmax + j];
                if (s >= 0 && s < K)
                    memcpy((char*)pool + ((size_t)unit * K + s) * rec_elems * es, rec,
                           rec_elems * es);
            }
            /* summary of block j over its tokens 0..u */
            size_t sbase = ((size_t)unit * NBmax + j) * 2 * (size_t)d;
            for (int c = 0; c < d; ++c) {
                size_t imin = (size_t)c, imax = (size_t)c;
                double vmin = elem(rec, dtype, imin), vmax = vmin;
                for (int v = 1; v <= u; ++v) {
                    size_t i = (size_t)v * d + c;
                    double x = elem(rec, dtype, i);
                    if (x < vmin) { vmin = x; imin = i; }
                    if (x > vmax) { vmax = x; imax = i; }
                }
                memcpy((char*)summ + (sbase + c) * es, rec + imin * es, es);
                memcpy((char*)summ + (sbase + d + c) * es, rec + imax * es, es);
            }
        }
        ctx_len[b] = t + 1;
    }
}
