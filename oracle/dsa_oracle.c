/*
 * dsa_oracle.c - plain, slow, obviously correct CPU oracle for the DSA
 * prefill/decode path (indexer -> top-k -> absorbed-MLA attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no source,
 * header, table or helper with the HIP library, and neither includes the
 * other.
 *
 * Sources (the pages; section names, no line numbers):
 *  - exo PR #2539 "GLM-5.2/5.3 (glm_moe_dsa) attention and MoE speed-ups",
 *    Prefill section: the indexer score (weighted relu of q.k summed over the
 *    32 indexer heads, float32, causal mask applied), the top-2048 selection,
 *    the every-earlier-key rule for queries with fewer causal keys than the
 *    selection size, and the float32 softmax over gathered latent keys;
 *    Decode section: single-token attention with the heads as rows.
 *  - "GLM-5.2-Vision: llama.cpp vs vLLM line-by-line pipeline trace",
 *    section 6 (attention core, absorbed MLA): Q = [q_nope_absorbed | q_pe],
 *    K = [kv_cmpr | k_pe], V = kv_cmpr; kq = K.q, softmax with kq_scale,
 *    kqv = V.kq.  The config line gives index_topk 2048 and the head widths.
 *    Sections 4 and 5 (KV compression path, RoPE convention) define the
 *    upstream cache write at the end of this file.
 *
 * Readings where the pages are silent are stated at each function and in
 * the design notes: key j is visible to the query at position p iff j <= p;
 * equal scores go to the lower key index; the selection is returned in
 * ascending key order padded with -1; no extra factor enters the indexer.
 *
 * Every step is computed in double precision except where noted.  There is
 * no blocking, fusion or reordering beyond the definitions.
 */
#include "dsa_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- step 1: load and convert ------------------------------------------
 * bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double* widen_all(const uint16_t* src, int64_t n) {
    double* dst = (double*)malloc((size_t)n * sizeof(double));
    if (!dst) return NULL;
    for (int64_t k = 0; k < n; ++k) dst[k] = bf16_to_double(src[k]);
    return dst;
}

/* ---- a plain parallel-for over rows: row r goes to thread r % T --------- */
typedef void (*row_fn)(void* ctx, int64_t r, void* scratch);

typedef struct {
    row_fn fn;
    void* ctx;
    int64_t nrows;
    int32_t tid, nthreads;
    size_t scratch_bytes;
    int failed;
} pf_job;

static void* pf_worker(void* arg) {
    pf_job* j = (pf_job*)arg;
    void* scratch = NULL;
    if (j->scratch_bytes) {
        scratch = malloc(j->scratch_bytes);
        if (!scratch) { j->failed = 1; return NULL; }
    }
    for (int64_t r = j->tid; r < j->nrows; r += j->nthreads) j->fn(j->ctx, r, scratch);
    free(scratch);
    return NULL;
}

static int parallel_rows(row_fn fn, void* ctx, int64_t nrows, int32_t nthreads, size_t scratch_bytes) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nrows) nthreads = (int32_t)(nrows > 0 ? nrows : 1);
    pthread_t th[256];
    pf_job jobs[256];
    int started[256];
    for (int32_t t = 0; t < nthreads; ++t) {
        jobs[t] = (pf_job){fn, ctx, nrows, t, nthreads, scratch_bytes, 0};
        started[t] = (t > 0) && pthread_create(&th[t], NULL, pf_worker, &jobs[t]) == 0;
    }
    pf_worker(&jobs[0]);
    int failed = jobs[0].failed;
    for (int32_t t = 1; t < nthreads; ++t) {
        if (started[t]) pthread_join(th[t], NULL);
        else pf_worker(&jobs[t]);          /* could not start a thread: run inline */
        failed |= jobs[t].failed;
    }
    return failed ? -9 : 0;
}

/* ---- step 2: indexer scores ---------------------------------------------
 * exo PR #2539, Prefill section, float32 indexer item: the per-key score is
 * relu(q.k) times each head's weight, summed over the indexer heads, with the
 * causal mask applied.  One Di-wide indexer key per token is shared by all
 * heads; w is per query and head; nothing else scales the sum. */
static void indexer_row(const double* qIrow /* [Hi*Di] */, const double* kId /* [N*Di] */,
                        const float* wrow /* [Hi] */, int64_t N, int64_t p,
                        int32_t Hi, int32_t Di, float* Srow) {
    for (int64_t j = 0; j < N; ++j) {
        if (j > p) { Srow[j] = -INFINITY; continue; }     /* causal mask */
        double total = 0.0;
        for (int32_t h = 0; h < Hi; ++h) {
            double dot = 0.0;
            for (int32_t d = 0; d < Di; ++d) dot += qIrow[(int64_t)h * Di + d] * kId[j * Di + d];
            double relu = dot > 0.0 ? dot : 0.0;
            total += (double)wrow[h] * relu;
        }
        Srow[j] = (float)total;   /* the pages' score is a float32 value */
    }
}

typedef struct {
    const uint16_t* qI; const double* kId; const float* w;
    int64_t N, q_start; int32_t Hi, Di;
    const int64_t* rows; float* S_out;
} indexer_ctx;

static void indexer_task(void* c, int64_t r, void* scratch) {
    indexer_ctx* x = (indexer_ctx*)c;
    int64_t i = x->rows[r];
    double* qrow = (double*)scratch;
    const uint16_t* src = x->qI + i * (int64_t)x->Hi * x->Di;
    for (int64_t k = 0; k < (int64_t)x->Hi * x->Di; ++k) qrow[k] = bf16_to_double(src[k]);
    indexer_row(qrow, x->kId, x->w + i * x->Hi, x->N, x->q_start + i, x->Hi, x->Di,
                x->S_out + r * x->N);
}

static int rows_ok(const int64_t* rows, int64_t nrows, int64_t L) {
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= L) return 0;
    return 1;
}

int oracle_indexer_scores(const uint16_t* qI, const uint16_t* kI, const float* w,
                          int64_t L, int64_t N, int64_t q_start, int32_t Hi, int32_t Di,
                          const int64_t* rows, int64_t nrows, float* S_out, int32_t nthreads) {
    if (!qI || !kI || !w || !rows || !S_out) return -1;
    if (L <= 0 || N <= 0 || Hi <= 0 || Di <= 0 || nrows < 0 || q_start < 0) return -1;
    if (!rows_ok(rows, nrows, L)) return -1;
    double* kId = widen_all(kI, N * Di);
    if (!kId) return -8;
    indexer_ctx x = {qI, kId, w, N, q_start, Hi, Di, rows, S_out};
    int rc = parallel_rows(indexer_task, &x, nrows, nthreads, (size_t)Hi * Di * sizeof(double));
    free(kId);
    return rc;
}

/* ---- step 3: top-k selection --------------------------------------------
 * exo PR #2539, Prefill section: each query keeps its index_topk (2048)
 * highest-scoring causal keys; a query with no more causal keys than that
 * keeps every earlier key.  Readings: equal scores go to the lower key index;
 * the kept keys are listed in ascending key order and padded with -1. */
typedef struct { float s; int32_t j; } cand;

static int by_score_then_key(const void* a, const void* b) {
    const cand* x = (const cand*)a;
    const cand* y = (const cand*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int ascending_int(const void* a, const void* b) {
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return (x < y) ? -1 : (x > y);
}

static void topk_row(const float* Srow, int64_t p, int32_t top_k, cand* work,
                     int32_t* idxrow, int32_t* count) {
    int64_t n = p + 1;                       /* causal keys 0..p */
    for (int32_t t = 0; t < top_k; ++t) idxrow[t] = -1;
    if (n <= top_k) {                        /* every earlier key */
        for (int64_t j = 0; j < n; ++j) idxrow[j] = (int32_t)j;
        *count = (int32_t)n;
        return;
    }
    for (int64_t j = 0; j < n; ++j) { work[j].s = Srow[j]; work[j].j = (int32_t)j; }
    qsort(work, (size_t)n, sizeof(cand), by_score_then_key);
    for (int32_t t = 0; t < top_k; ++t) idxrow[t] = work[t].j;
    qsort(idxrow, (size_t)top_k, sizeof(int32_t), ascending_int);
    *count = top_k;
}

typedef struct {
    const float* S; int64_t N; const int64_t* pos; int32_t top_k;
    int32_t* idx; int32_t* count; int bad;
} topk_ctx;

static void topk_task(void* c, int64_t r, void* scratch) {
    topk_ctx* x = (topk_ctx*)c;
    topk_row(x->S + r * x->N, x->pos[r], x->top_k, (cand*)scratch,
             x->idx + r * x->top_k, x->count + r);
}

int oracle_topk_select(const float* S, int64_t nrows, int64_t N, const int64_t* pos,
                       int32_t top_k, int32_t* idx, int32_t* count, int32_t nthreads) {
    if (!S || !pos || !idx || !count || nrows < 0 || N <= 0 || top_k <= 0) return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (pos[r] < 0 || pos[r] >= N) return -1;
    topk_ctx x = {S, N, pos, top_k, idx, count, 0};
    return parallel_rows(topk_task, &x, nrows, nthreads, (size_t)N * sizeof(cand));
}

/* ---- step 4: absorbed-MLA attention over the selected latent rows --------
 * Pipeline trace, section 6: Q = [q_nope_absorbed | q_pe] (Dl + Dr wide),
 * K = [kv_cmpr | k_pe], V = kv_cmpr (the first Dl columns of the latent row);
 * scores K.q scaled by kq_scale, softmax, then V weighted by it.
 * exo PR #2539, Prefill section: the softmax runs over the gathered selected
 * keys only.  No bias, sink or soft-cap enters the softmax. */
static void attention_row(const double* qrow /* [H*Dqk] */, const double* kvd /* [N*Dqk] */,
                          const int32_t* sel, int32_t cnt, int64_t N, int32_t H, int32_t Dqk,
                          int32_t Dv, double scale, double* s /* [cnt] */,
                          double* outrow /* [H*Dv] */, double* lserow /* [H] or NULL */) {
    for (int32_t h = 0; h < H; ++h) {
        const double* qh = qrow + (int64_t)h * Dqk;
        double* oh = outrow + (int64_t)h * Dv;
        for (int32_t d = 0; d < Dv; ++d) oh[d] = 0.0;
        int32_t used = 0;
        double m = -INFINITY;
        for (int32_t t = 0; t < cnt; ++t) {
            int64_t j = sel[t];
            if (j < 0 || j >= N) { s[t] = -INFINITY; continue; }   /* not a key */
            double dot = 0.0;
            for (int32_t d = 0; d < Dqk; ++d) dot += qh[d] * kvd[j * Dqk + d];
            s[t] = scale * dot;
            if (s[t] > m) m = s[t];
            ++used;
        }
        if (used == 0) { if (lserow) lserow[h] = -INFINITY; continue; }
        double Z = 0.0;
        for (int32_t t = 0; t < cnt; ++t) Z += (s[t] == -INFINITY) ? 0.0 : exp(s[t] - m);
        for (int32_t t = 0; t < cnt; ++t) {
            if (s[t] == -INFINITY) continue;
            double pt = exp(s[t] - m) / Z;
            const double* v = kvd + (int64_t)sel[t] * Dqk;          /* V = first Dv columns */
            for (int32_t d = 0; d < Dv; ++d) oh[d] += pt * v[d];
        }
        if (lserow) lserow[h] = m + log(Z);
    }
}

typedef struct {
    const uint16_t* q; const double* kvd; const int32_t* idx; const int32_t* count;
    int64_t N; int32_t H, Dqk, Dv, top_k; double scale;
    const int64_t* rows; double* out; double* lse;
} attn_ctx;

static void attn_task(void* c, int64_t r, void* scratch) {
    attn_ctx* x = (attn_ctx*)c;
    int64_t i = x->rows[r];
    double* qrow = (double*)scratch;
    double* s = qrow + (int64_t)x->H * x->Dqk;
    const uint16_t* src = x->q + i * (int64_t)x->H * x->Dqk;
    for (int64_t k = 0; k < (int64_t)x->H * x->Dqk; ++k) qrow[k] = bf16_to_double(src[k]);
    int32_t cnt = x->count[i];
    if (cnt > x->top_k) cnt = x->top_k;
    attention_row(qrow, x->kvd, x->idx + i * x->top_k, cnt, x->N, x->H, x->Dqk, x->Dv, x->scale,
                  s, x->out + r * (int64_t)x->H * x->Dv, x->lse ? x->lse + r * x->H : NULL);
}

int oracle_sparse_mla_attn(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                           const int32_t* count, int64_t L, int64_t N, int32_t H, int32_t Dqk,
                           int32_t Dv, int32_t top_k, double scale,
                           const int64_t* rows, int64_t nrows, double* out, double* lse,
                           int32_t nthreads) {
    if (!q || !kv || !idx || !count || !rows || !out) return -1;
    if (L <= 0 || N <= 0 || H <= 0 || Dqk <= 0 || Dv <= 0 || Dv > Dqk || top_k <= 0 || nrows < 0)
        return -1;
    if (!rows_ok(rows, nrows, L)) return -1;
    double* kvd = widen_all(kv, N * Dqk);
    if (!kvd) return -8;
    attn_ctx x = {q, kvd, idx, count, N, H, Dqk, Dv, top_k, scale, rows, out, lse};
    int rc = parallel_rows(attn_task, &x, nrows, nthreads,
                           ((size_t)H * Dqk + (size_t)top_k) * sizeof(double));
    free(kvd);
    return rc;
}

/* ---- step 5: the chunk and the decode step end to end --------------------
 * exo PR #2539, Prefill section: queries with no more causal keys than the
 * selection size skip the indexer and take every earlier key; the others are
 * scored, selected and attended sparsely.  Decode section: a decode step is
 * one query per sequence at the end of its cache. */
typedef struct {
    const uint16_t *q, *qI; const float* w; const double *kvd, *kId;
    int64_t N, q_start; int32_t H, Dqk, Dv, Hi, Di, top_k; double scale;
    const int64_t* rows; int32_t* idx_out; int32_t* count_out; double* out;
} chunk_ctx;

static void chunk_task(void* c, int64_t r, void* scratch) {
    chunk_ctx* x = (chunk_ctx*)c;
    int64_t i = x->rows[r];
    int64_t p = x->q_start + i;
    /* scratch: S row [N] float | cand [N] | q row doubles | s [top_k] doubles */
    char* base = (char*)scratch;
    float* Srow = (float*)base;
    cand* work = (cand*)(base + (size_t)x->N * sizeof(float));
    double* qrow = (double*)(base + (size_t)x->N * (sizeof(float) + sizeof(cand)));
    int64_t qw = (int64_t)x->Hi * x->Di > (int64_t)x->H * x->Dqk ? (int64_t)x->Hi * x->Di
                                                                 : (int64_t)x->H * x->Dqk;
    double* s = qrow + qw;
    int32_t* sel = x->idx_out + r * x->top_k;
    if (p + 1 > x->top_k) {
        const uint16_t* src = x->qI + i * (int64_t)x->Hi * x->Di;
        for (int64_t k = 0; k < (int64_t)x->Hi * x->Di; ++k) qrow[k] = bf16_to_double(src[k]);
        indexer_row(qrow, x->kId, x->w + i * x->Hi, x->N, p, x->Hi, x->Di, Srow);
    }
    topk_row(Srow, p, x->top_k, work, sel, x->count_out + r);
    const uint16_t* src = x->q + i * (int64_t)x->H * x->Dqk;
    for (int64_t k = 0; k < (int64_t)x->H * x->Dqk; ++k) qrow[k] = bf16_to_double(src[k]);
    attention_row(qrow, x->kvd, sel, x->count_out[r], x->N, x->H, x->Dqk, x->Dv, x->scale, s,
                  x->out + r * (int64_t)x->H * x->Dv, NULL);
}

static size_t chunk_scratch(int64_t N, int32_t H, int32_t Dqk, int32_t Hi, int32_t Di, int32_t top_k) {
    int64_t qw = (int64_t)Hi * Di > (int64_t)H * Dqk ? (int64_t)Hi * Di : (int64_t)H * Dqk;
    return (size_t)N * (sizeof(float) + sizeof(cand)) + ((size_t)qw + (size_t)top_k) * sizeof(double);
}

int oracle_prefill_chunk(const uint16_t* q, const uint16_t* qI, const float* w,
                         const uint16_t* kv, const uint16_t* kI,
                         int64_t L, int64_t N, int64_t q_start,
                         int32_t H, int32_t Dl, int32_t Dr, int32_t Hi, int32_t Di,
                         int32_t top_k, double scale,
                         const int64_t* rows, int64_t nrows,
                         int32_t* idx_out, int32_t* count_out, double* out, int32_t nthreads) {
    if (!q || !qI || !w || !kv || !kI || !rows || !idx_out || !count_out || !out) return -1;
    if (L <= 0 || N <= 0 || q_start < 0 || q_start + L > N || H <= 0 || Dl <= 0 || Dr < 0 ||
        Hi <= 0 || Di <= 0 || top_k <= 0 || nrows < 0)
        return -1;
    if (!rows_ok(rows, nrows, L)) return -1;
    int32_t Dqk = Dl + Dr;
    double* kvd = widen_all(kv, N * Dqk);
    double* kId = widen_all(kI, N * Di);
    if (!kvd || !kId) { free(kvd); free(kId); return -8; }
    chunk_ctx x = {q, qI, w, kvd, kId, N, q_start, H, Dqk, Dl, Hi, Di, top_k, scale,
                   rows, idx_out, count_out, out};
    int rc = parallel_rows(chunk_task, &x, nrows, nthreads, chunk_scratch(N, H, Dqk, Hi, Di, top_k));
    free(kvd);
    free(kId);
    return rc;
}

int oracle_decode_step(const uint16_t* q, const uint16_t* qI, const float* w,
                       const uint16_t* kv, const uint16_t* kI, int32_t B, const int64_t* ctx,
                       int32_t H, int32_t Dl, int32_t Dr, int32_t Hi, int32_t Di,
                       int32_t top_k, double scale,
                       int32_t* idx_out, int32_t* count_out, double* out, int32_t nthreads) {
    if (!q || !qI || !w || !kv || !kI || !ctx || !idx_out || !count_out || !out || B <= 0) return -1;
    int32_t Dqk = Dl + Dr;
    int64_t off = 0;
    for (int32_t b = 0; b < B; ++b) {
        if (ctx[b] <= 0) return -1;
        /* sequence b is a one-query chunk at position ctx-1 over its own cache */
        int64_t row0 = 0;
        int rc = oracle_prefill_chunk(q + (int64_t)b * H * Dqk, qI + (int64_t)b * Hi * Di, w + (int64_t)b * Hi,
                                      kv + off * Dqk, kI + off * Di, 1, ctx[b], ctx[b] - 1,
                                      H, Dl, Dr, Hi, Di, top_k, scale, &row0, 1,
                                      idx_out + (int64_t)b * top_k, count_out + b,
                                      out + (int64_t)b * H * Dl, nthreads);
        if (rc) return rc;
        off += ctx[b];
    }
    return 0;
}

/* ==========================================================================
 * Upstream cache write ("GLM-5.2-Vision: llama.cpp vs vLLM" pipeline trace,
 * section 4, KV compression path, and section 5, RoPE convention): the kv_a
 * projection output of a token is split into kv_cmpr (the first Dl columns)
 * and k_pe (the last Dr); k_pe and the query's q_pe are rotated by RoPE of
 * the NORM flavour (adjacent pairs x[2i], x[2i+1]); kv_cmpr is RMS-normalised
 * and scaled by the kv_a norm weight after the split; the indexer's query
 * and key are rotated the same way (the trace's note that the indexer rope
 * is NORM too).  Readings: the rotation angle of pair i over a rope width d
 * at position p is p * theta^(-2i/d) (theta is not on the pages and is an
 * argument); the indexer rope covers the first d_idx_rope columns of each
 * indexer head; RMSNorm is x / sqrt(mean(x^2) + eps) * weight.
 * ======================================================================== */

/* double -> bf16 bits, round to nearest with ties to even, for zero and
 * values in the normal bf16 range: keep 8 significant bits. */
static uint16_t double_to_bf16(double v) {
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    int e;
    double m = frexp(fabs(v), &e);          /* |v| = m * 2^e, m in [0.5, 1) */
    double r = nearbyint(ldexp(m, 8));      /* default rounding: ties to even */
    float f = (float)ldexp(signbit(v) ? -r : r, e - 8);   /* exact: 8 bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* RoPE, NORM flavour, in place on x[0..d): pair (x[2i], x[2i+1]) turns by
 * the angle p * theta^(-2i/d). */
static void rope_norm(double* x, int32_t d, double p, double theta) {
    for (int32_t i = 0; i < d / 2; ++i) {
        double ang = p * pow(theta, -2.0 * i / d);
        double c = cos(ang), s = sin(ang);
        double a = x[2 * i], b = x[2 * i + 1];
        x[2 * i] = a * c - b * s;
        x[2 * i + 1] = a * s + b * c;
    }
}

/* RMSNorm in place on x[0..n): x / sqrt(mean(x^2) + eps) * w. */
static void rms_norm(double* x, int32_t n, const float* w, double eps) {
    double ss = 0.0;
    for (int32_t k = 0; k < n; ++k) ss += x[k] * x[k];
    double r = 1.0 / sqrt(ss / n + eps);
    for (int32_t k = 0; k < n; ++k) x[k] = x[k] * r * (double)w[k];
}

/* Rope the first `d` of the `width` columns of each of `nheads` bf16 rows
 * (in place, rounded once to bf16). */
static void rope_rows_bf16(uint16_t* rows, int32_t nheads, int32_t width, int32_t col0, int32_t d,
                           double p, double theta, double* tmp) {
    for (int32_t h = 0; h < nheads; ++h) {
        uint16_t* r = rows + (int64_t)h * width + col0;
        for (int32_t k = 0; k < d; ++k) tmp[k] = bf16_to_double(r[k]);
        rope_norm(tmp, d, p, theta);
        for (int32_t k = 0; k < d; ++k) r[k] = double_to_bf16(tmp[k]);
    }
}

int oracle_cache_write(const uint16_t* kv_a, const float* norm_w, double eps,
                       const int64_t* pos, int64_t T, int64_t N,
                       uint16_t* kv_cache, const uint16_t* kI_new, uint16_t* kI_cache,
                       uint16_t* q, uint16_t* qI,
                       int32_t H, int32_t Dl, int32_t Dr, int32_t Hi, int32_t Di,
                       int32_t d_idx_rope, double theta) {
    if (!kv_a || !norm_w || !pos || !kv_cache || T < 0 || N <= 0 || H <= 0 || Dl <= 0 ||
        Dr < 0 || (Dr & 1) || Hi <= 0 || Di <= 0 || d_idx_rope < 0 || (d_idx_rope & 1) ||
        d_idx_rope > Di || !(theta > 0.0) || !(eps >= 0.0) || (!kI_new) != (!kI_cache))
        return -1;
    int32_t Dqk = Dl + Dr;
    int32_t wmax = Dqk > Di ? Dqk : Di;
    double* tmp = (double*)malloc((size_t)wmax * sizeof(double));
    if (!tmp) return -8;
    for (int64_t t = 0; t < T; ++t) {
        double p = (double)pos[t];
        if (pos[t] >= 0 && pos[t] < N) {
            /* latent cache row: [rmsnorm(kv_cmpr) * w | rope(k_pe)] */
            const uint16_t* src = kv_a + t * Dqk;
            uint16_t* dst = kv_cache + pos[t] * Dqk;
            for (int32_t k = 0; k < Dqk; ++k) tmp[k] = bf16_to_double(src[k]);
            rms_norm(tmp, Dl, norm_w, eps);
            rope_norm(tmp + Dl, Dr, p, theta);
            for (int32_t k = 0; k < Dqk; ++k) dst[k] = double_to_bf16(tmp[k]);
            /* indexer cache row: the new key with its leading columns roped */
            if (kI_new) {
                const uint16_t* ks = kI_new + t * Di;
                uint16_t* kd = kI_cache + pos[t] * Di;
                for (int32_t k = 0; k < Di; ++k) tmp[k] = bf16_to_double(ks[k]);
                rope_norm(tmp, d_idx_rope, p, theta);
                for (int32_t k = 0; k < Di; ++k) kd[k] = double_to_bf16(tmp[k]);
            }
        }
        /* the query's rope part of every head, and the indexer query */
        if (q) rope_rows_bf16(q + t * H * Dqk, H, Dqk, Dl, Dr, p, theta, tmp);
        if (qI) rope_rows_bf16(qI + t * Hi * Di, Hi, Di, 0, d_idx_rope, p, theta, tmp);
    }
    free(tmp);
    return 0;
}

/* ==========================================================================
 * Router selection ("GLM-5.2-Vision: llama.cpp vs vLLM" pipeline trace,
 * section 8a, Gating; exo PR #2539, router selection in one kernel): per
 * token the expert probabilities are the sigmoid of the float32 router
 * logits; the selection score adds the per-expert bias, which is used for
 * the choice only; the k best experts by selection score are kept; their
 * weights are the unbiased probabilities divided by their sum (clamped
 * below at 6.1e-5) and multiplied by the routed scaling factor (GLM: 256
 * experts, 8 per token, factor 2.5, one expert group).  Readings: a float32
 * probability is the exact sigmoid rounded once to float; the selection
 * score is that float plus the bias in float arithmetic; equal selection
 * scores go to the lower expert index; experts are listed by descending
 * selection score.
 * ======================================================================== */
typedef struct { float s; int32_t e; } expert_key;

static int by_score_then_index(const void* a, const void* b) {
    const expert_key* x = (const expert_key*)a;
    const expert_key* y = (const expert_key*)b;
    if (x->s != y->s) return x->s > y->s ? -1 : 1;   /* higher selection score first */
    return (x->e < y->e) ? -1 : (x->e > y->e);
}

int oracle_router_topk(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
                       double scale, double min_sum, int32_t* ids, double* weights) {
    if (!logits || !bias || !ids || !weights || T < 0 || E <= 0 || k <= 0 || k > E) return -1;
    float* p = (float*)malloc((size_t)E * sizeof(float));
    expert_key* key = (expert_key*)malloc((size_t)E * sizeof(expert_key));
    if (!p || !key) { free(p); free(key); return -8; }
    for (int64_t t = 0; t < T; ++t) {
        const float* lg = logits + t * E;
        for (int32_t e = 0; e < E; ++e) {
            p[e] = (float)(1.0 / (1.0 + exp(-(double)lg[e])));
            key[e].s = p[e] + bias[e];            /* float + float, rounded to float */
            key[e].e = e;
        }
        qsort(key, (size_t)E, sizeof(expert_key), by_score_then_index);
        double sum = 0.0;
        for (int32_t j = 0; j < k; ++j) sum += (double)p[key[j].e];
        double den = sum > min_sum ? sum : min_sum;
        for (int32_t j = 0; j < k; ++j) {
            ids[t * k + j] = key[j].e;
            weights[t * k + j] = (double)p[key[j].e] / den * scale;
        }
    }
    free(p);
    free(key);
    return 0;
}

/* ==========================================================================
 * Downstream projections ("GLM-5.2-Vision: llama.cpp vs vLLM" pipeline
 * trace, section 6, build_attn: the attention output in the latent space is
 * decompressed per head with wv_b, kqv = v_mla . kqv, then flattened over the
 * heads and multiplied by the output projection wo; the config line gives
 * v_head_dim 256 and hidden 6144).  Readings: weights are stored as
 * [out, in] (bf16, in-dimension contiguous); the products take bf16
 * operands, so the float32 attention output is rounded once to bf16 and the
 * up-projected values are rounded once to bf16 before the output
 * projection; sums are exact here (double).
 * ======================================================================== */

/* out_v[t, h, j] = bf16( sum_c bf16(o[t, h, c]) * wv[h, j, c] ),
 *   o [T, H, Dl] float, wv [H, Dv, Dl] bf16, out_v [T, H, Dv] bf16. */
int oracle_value_up_proj(const float* o, const uint16_t* wv, int64_t T, int32_t H, int32_t Dl,
                         int32_t Dv, uint16_t* out_v) {
    if (!o || !wv || !out_v || T < 0 || H <= 0 || Dl <= 0 || Dv <= 0) return -1;
    double* x = (double*)malloc((size_t)Dl * sizeof(double));
    if (!x) return -8;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            const float* orow = o + (t * H + h) * Dl;
            for (int32_t c = 0; c < Dl; ++c) x[c] = bf16_to_double(double_to_bf16((double)orow[c]));
            for (int32_t j = 0; j < Dv; ++j) {
                const uint16_t* wrow = wv + ((int64_t)h * Dv + j) * Dl;
                double acc = 0.0;
                for (int32_t c = 0; c < Dl; ++c) acc += x[c] * bf16_to_double(wrow[c]);
                out_v[(t * H + h) * Dv + j] = double_to_bf16(acc);
            }
        }
    }
    free(x);
    return 0;
}

/* y[t, n] = sum_k x[t, k] * wo[n, k],  x [T, Kin] bf16, wo [Nout, Kin] bf16,
 * y [T, Nout] double. */
int oracle_o_proj(const uint16_t* x, const uint16_t* wo, int64_t T, int32_t Kin, int32_t Nout,
                  const int64_t* rows, int64_t nrows, double* y) {
    if (!x || !wo || !y || T < 0 || Kin <= 0 || Nout <= 0 || nrows < 0) return -1;
    double* xr = (double*)malloc((size_t)Kin * sizeof(double));
    if (!xr) return -8;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t t = rows ? rows[r] : r;
        if (t < 0 || t >= T) { free(xr); return -1; }
        for (int32_t k = 0; k < Kin; ++k) xr[k] = bf16_to_double(x[t * Kin + k]);
        for (int32_t n = 0; n < Nout; ++n) {
            const uint16_t* wrow = wo + (int64_t)n * Kin;
            double acc = 0.0;
            for (int32_t k = 0; k < Kin; ++k) acc += xr[k] * bf16_to_double(wrow[k]);
            y[r * Nout + n] = acc;
        }
    }
    free(xr);
    return 0;
}

/* ==========================================================================
 * Dense masked attention in the non-absorbed form (exo PR #2539, Prefill
 * section, dense attention in one product: below 8192 keys of context each
 * head's 192 no-rope and 64 rope dimensions are scored in one 256-wide
 * product under a boolean mask).  The head widths come from the config line
 * of the pipeline trace (qk_nope 192, qk_rope 64, v_head_dim 256); section 4
 * of the trace splits the kv_b output per head into the no-rope key and the
 * value, and the rope key is the one shared k_pe of the cache row.
 * Readings: the boolean mask is the query's DSA selection (for a query with
 * no more causal keys than top_k that is every earlier key), restricted to
 * causal keys j <= p; the scale is the one the absorbed form uses.
 * ======================================================================== */

/* mask[i, w] bit b set iff key 32 w + b is among idx[i, :count[i]], lies in
 * [0, N) and is causal for the query at position q_start + i.
 * mask [L, W] uint32 with W >= ceil(N / 32); bits at or past N stay 0. */
int oracle_selection_mask(const int32_t* idx, const int32_t* count, int64_t L, int32_t top_k,
                          int64_t N, int64_t q_start, int64_t W, uint32_t* mask) {
    if (!idx || !count || !mask || L < 0 || top_k <= 0 || N <= 0 || W * 32 < N) return -1;
    for (int64_t i = 0; i < L; ++i) {
        uint32_t* row = mask + i * W;
        for (int64_t w = 0; w < W; ++w) row[w] = 0u;
        const int64_t p = q_start + i;
        int32_t c = count[i];
        if (c < 0) c = 0;
        if (c > top_k) c = top_k;
        for (int32_t t = 0; t < c; ++t) {
            const int64_t j = idx[i * top_k + t];
            if (j >= 0 && j < N && j <= p) row[j / 32] |= 1u << (j % 32);
        }
    }
    return 0;
}

typedef struct {
    const uint16_t *q, *kvb, *kv; const uint32_t* mask;
    int64_t N, W; int32_t H, Dn, Dr, Dv, Dc, rope_col; double scale;
    const int64_t* rows; double* out;
} dense_ctx;

/* One query, every head: s_j = scale * (q_nope . k_nope_j + q_pe . k_pe_j)
 * over the keys the mask holds, softmax, out = sum_j p_j v_j. */
static void dense_task(void* c, int64_t r, void* scratch) {
    dense_ctx* x = (dense_ctx*)c;
    const int64_t i = x->rows[r];
    double* s = (double*)scratch;                                /* [N] */
    const uint32_t* mrow = x->mask + i * x->W;
    const int32_t Dq = x->Dn + x->Dr, Dkv = x->Dn + x->Dv;
    for (int32_t h = 0; h < x->H; ++h) {
        const uint16_t* qh = x->q + (i * x->H + h) * Dq;
        double* oh = x->out + (r * x->H + h) * x->Dv;
        for (int32_t e = 0; e < x->Dv; ++e) oh[e] = 0.0;
        double m = -INFINITY;
        for (int64_t j = 0; j < x->N; ++j) {
            if (!((mrow[j / 32] >> (j % 32)) & 1u)) { s[j] = -INFINITY; continue; }
            const uint16_t* kn = x->kvb + (j * x->H + h) * Dkv;        /* no-rope key of head h */
            const uint16_t* kp = x->kv + j * x->Dc + x->rope_col;      /* shared rope key */
            double dot = 0.0;
            for (int32_t d = 0; d < x->Dn; ++d) dot += bf16_to_double(qh[d]) * bf16_to_double(kn[d]);
            for (int32_t d = 0; d < x->Dr; ++d) dot += bf16_to_double(qh[x->Dn + d]) * bf16_to_double(kp[d]);
            s[j] = x->scale * dot;
            if (s[j] > m) m = s[j];
        }
        if (m == -INFINITY) continue;                              /* no key: zeros */
        double Z = 0.0;
        for (int64_t j = 0; j < x->N; ++j)
            if (s[j] != -INFINITY) Z += exp(s[j] - m);
        for (int64_t j = 0; j < x->N; ++j) {
            if (s[j] == -INFINITY) continue;
            const double pj = exp(s[j] - m) / Z;
            const uint16_t* v = x->kvb + (j * x->H + h) * Dkv + x->Dn;  /* value of head h */
            for (int32_t e = 0; e < x->Dv; ++e) oh[e] += pj * bf16_to_double(v[e]);
        }
    }
}

int oracle_dense_masked_attn(const uint16_t* q, const uint16_t* kvb, const uint16_t* kv,
                             const uint32_t* mask, int64_t L, int64_t N, int32_t H, int32_t Dn,
                             int32_t Dr, int32_t Dv, int32_t Dc, int32_t rope_col, int64_t W,
                             double scale, const int64_t* rows, int64_t nrows, double* out,
                             int32_t nthreads) {
    if (!q || !kvb || !kv || !mask || !rows || !out) return -1;
    if (L <= 0 || N <= 0 || H <= 0 || Dn < 0 || Dr < 0 || Dv <= 0 || rope_col < 0 ||
        rope_col + Dr > Dc || W * 32 < N || nrows < 0)
        return -1;
    if (!rows_ok(rows, nrows, L)) return -1;
    dense_ctx x = {q, kvb, kv, mask, N, W, H, Dn, Dr, Dv, Dc, rope_col, scale, rows, out};
    return parallel_rows(dense_task, &x, nrows, nthreads, (size_t)N * sizeof(double));
}

/* ==========================================================================
 * The kv_b up-projection of the dense path (pipeline trace, section 4: the
 * kv_b projection of the normalised latent gives, per head, the no-rope key
 * and the value; config line: qk_nope 192, v_head_dim 256).  Readings: the
 * weight is stored [H * (Dn + Dv), Dl] ([out, in]); the latent is the first
 * Dl columns of each cache row; the sums are exact here (double) and each
 * result is rounded once, to bf16 for the no-rope key columns and, when
 * values_f16 is set, to fp16 for the value columns (the form the dense
 * attention's value product reads).
 * ======================================================================== */

/* double -> IEEE binary16 bits, round to nearest with ties to even;
 * magnitudes from 65520 up become infinities. */
static uint16_t double_to_f16(double v) {
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    const double m = frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1;                                  /* a = (2m) * 2^E */
    if (E < -14) {                                  /* subnormal: spacing 2^-24 */
        const double n = nearbyint(ldexp(a, 24));   /* 1024 lands on the smallest normal */
        return (uint16_t)(sign | (uint16_t)n);
    }
    double n = nearbyint(ldexp(m, 11));             /* 11 significant bits, in [1024, 2048] */
    if (n == 2048.0) { n = 1024.0; ++E; }
    if (E > 15) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0));
}

/* kvb[j, h, c] = round( sum_d kv[j, d] * w[h * (Dn + Dv) + c, d] ),  d < Dl. */
int oracle_kv_b_proj(const uint16_t* kv, int32_t kv_cols, const uint16_t* w, int64_t N, int32_t H,
                     int32_t Dl, int32_t Dn, int32_t Dv, int32_t values_f16, uint16_t* kvb) {
    if (!kv || !w || !kvb || N < 0 || H <= 0 || Dl <= 0 || Dl > kv_cols || Dn < 0 || Dv <= 0) return -1;
    const int32_t C = Dn + Dv;
    double* x = (double*)malloc((size_t)Dl * sizeof(double));
    if (!x) return -8;
    for (int64_t j = 0; j < N; ++j) {
        for (int32_t d = 0; d < Dl; ++d) x[d] = bf16_to_double(kv[j * kv_cols + d]);
        for (int32_t h = 0; h < H; ++h) {
            for (int32_t c = 0; c < C; ++c) {
                const uint16_t* wrow = w + ((int64_t)h * C + c) * Dl;
                double acc = 0.0;
                for (int32_t d = 0; d < Dl; ++d) acc += x[d] * bf16_to_double(wrow[d]);
                kvb[(j * H + h) * C + c] = (values_f16 && c >= Dn) ? double_to_f16(acc) : double_to_bf16(acc);
            }
        }
    }
    free(x);
    return 0;
}

/* Query absorption, "GLM-5.2-Vision: llama.cpp vs vLLM line-by-line pipeline
 * trace", section 6: each head's no-rope query is carried into the latent
 * space through the key block of the kv_b weight, so that it can score the
 * shared latent rows directly.  With C = Dn + Dv:
 *   out[t, h, d]      = round( sum_c q[t, h, c] * w[h*C + c, d] ),  c < Dn, d < Dl
 *   out[t, h, Dl + r] = q[t, h, Dn + r]                            (the rope part, copied)
 * q [T, H, Dn + Dr] bf16, w [H*C, Dl] bf16 (the kv_b weight), out
 * [T, H, Dl + Dr] bf16 (nearest even).  For every latent row kv,
 * <out[t, h, :Dl], kv> equals <q[t, h, :Dn], kvb key> before the rounding. */
int oracle_q_absorb(const uint16_t* q, const uint16_t* w, int64_t T, int32_t H, int32_t Dn, int32_t Dr,
                    int32_t Dl, int32_t Dv, uint16_t* out) {
    if (!q || !w || !out || T < 0 || H <= 0 || Dn <= 0 || Dr < 0 || Dl <= 0 || Dv < 0) return -1;
    const int32_t C = Dn + Dv;
    double* qn = (double*)malloc((size_t)Dn * sizeof(double));
    if (!qn) return -8;
    for (int64_t t = 0; t < T; ++t) {
        for (int32_t h = 0; h < H; ++h) {
            const uint16_t* qrow = q + (t * H + h) * (int64_t)(Dn + Dr);
            uint16_t* orow = out + (t * H + h) * (int64_t)(Dl + Dr);
            for (int32_t c = 0; c < Dn; ++c) qn[c] = bf16_to_double(qrow[c]);
            for (int32_t d = 0; d < Dl; ++d) {
                double acc = 0.0;
                for (int32_t c = 0; c < Dn; ++c) acc += qn[c] * bf16_to_double(w[((int64_t)h * C + c) * Dl + d]);
                orow[d] = double_to_bf16(acc);
            }
            for (int32_t r = 0; r < Dr; ++r) orow[Dl + r] = qrow[Dn + r];
        }
    }
    free(qn);
    return 0;
}
