/*
 * dsa_oracle.h - plain CPU oracle for the DeepSeek-sparse-attention (DSA)
 * prefill/decode path.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the benchmark's CPU-baseline leg call it; the HIP library never does,
 * and it shares no code, header, table or helper with the HIP library.
 *
 * Arithmetic: every floating-point step in double precision.  The one place
 * the pages fix a precision is the indexer score, which exo PR #2539 (Prefill
 * section, float32 indexer item) sums in float32; the oracle therefore forms
 * the exact score in double and rounds it once to float, and the top-k
 * decision compares those float values.
 *
 * Storage conventions (all arrays dense, row-major, host memory):
 *   bf16 operands are passed as uint16_t bit patterns;
 *   a prefill chunk has L queries at positions q_start + i over keys 0..N-1;
 *   key j is visible to the query at position p iff j <= p.
 *
 * Every function returns 0 on success and a negative value on a bad
 * argument (null pointer, non-positive size, row out of range).
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Indexer scores for selected query rows.
 *   qI [L, Hi, Di] bf16, kI [N, Di] bf16, w [L, Hi] float.
 *   rows[r] (r < nrows) names the query row; S_out is [nrows, N] float.
 * S_out[r, j] = float( sum_h w[i,h] * max(0, sum_d qI[i,h,d] * kI[j,d]) )
 * for j <= q_start + i, and -infinity for later keys. */
int oracle_indexer_scores(const uint16_t* qI, const uint16_t* kI, const float* w,
                          int64_t L, int64_t N, int64_t q_start, int32_t Hi, int32_t Di,
                          const int64_t* rows, int64_t nrows, float* S_out, int32_t nthreads);

/* Top-k selection for nrows score rows S [nrows, N]; pos[r] is the query's
 * position (keys 0..pos[r] are candidates, pos[r] < N).
 *   pos+1 <= top_k : idx = 0..pos (every earlier key, scores unused);
 *   otherwise      : the top_k keys ordered by (score descending, key
 *                    ascending), written in ascending key order.
 * idx [nrows, top_k] is padded with -1; count[r] = min(pos+1, top_k). */
int oracle_topk_select(const float* S, int64_t nrows, int64_t N, const int64_t* pos,
                       int32_t top_k, int32_t* idx, int32_t* count, int32_t nthreads);

/* Absorbed-MLA attention over selected latent rows.
 *   q [L, H, Dqk] bf16; kv [N, Dqk] bf16 (value = first Dv columns);
 *   idx [L, top_k] key ids (first count[i] used); rows[r] names the query.
 *   out [nrows, H, Dv] double; lse [nrows, H] double (may be NULL).
 * s_t = scale * <q[i,h,:], kv[idx_t,:]>;  out = sum_t softmax(s)_t kv[idx_t,:Dv];
 * lse = log sum_t exp(s_t).  count 0 gives out = 0, lse = -inf. */
int oracle_sparse_mla_attn(const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                           const int32_t* count, int64_t L, int64_t N, int32_t H, int32_t Dqk,
                           int32_t Dv, int32_t top_k, double scale,
                           const int64_t* rows, int64_t nrows, double* out, double* lse,
                           int32_t nthreads);

/* One prefill chunk end to end for selected rows: indexer (only for queries
 * with more causal keys than top_k), top-k, attention.
 * idx_out [nrows, top_k], count_out [nrows], out [nrows, H, Dv] (double). */
int oracle_prefill_chunk(const uint16_t* q, const uint16_t* qI, const float* w,
                         const uint16_t* kv, const uint16_t* kI,
                         int64_t L, int64_t N, int64_t q_start,
                         int32_t H, int32_t Dl, int32_t Dr, int32_t Hi, int32_t Di,
                         int32_t top_k, double scale,
                         const int64_t* rows, int64_t nrows,
                         int32_t* idx_out, int32_t* count_out, double* out, int32_t nthreads);

/* One batched decode step: B sequences, one query each at position ctx[b]-1,
 * caches packed in sequence order (sequence b's rows start at sum(ctx[:b])).
 *   q [B, H, Dl+Dr], qI [B, Hi, Di], w [B, Hi], kv [sum ctx, Dl+Dr], kI [sum ctx, Di].
 * idx_out [B, top_k] (key ids local to the sequence), count_out [B], out [B, H, Dl]. */
int oracle_decode_step(const uint16_t* q, const uint16_t* qI, const float* w,
                       const uint16_t* kv, const uint16_t* kI, int32_t B, const int64_t* ctx,
                       int32_t H, int32_t Dl, int32_t Dr, int32_t Hi, int32_t Di,
                       int32_t top_k, double scale,
                       int32_t* idx_out, int32_t* count_out, double* out, int32_t nthreads);

/* Upstream cache write for T new tokens (pipeline trace sections 4 and 5).
 *   kv_a [T, Dl+Dr] bf16: per token [kv_cmpr | k_pe] from the kv_a projection;
 *   norm_w [Dl] float, eps: the RMSNorm weight and epsilon;
 *   pos [T]: token positions; a token with 0 <= pos < N writes cache rows pos:
 *     kv_cache [N, Dl+Dr] bf16: [rmsnorm(kv_cmpr) * norm_w | rope(k_pe, pos)];
 *     kI_cache [N, Di] bf16: kI_new[t] with its first d_idx_rope columns
 *       roped (kI_new, kI_cache both NULL: skipped);
 *   q [T, H, Dl+Dr] bf16 or NULL: columns Dl.. of every head roped in place;
 *   qI [T, Hi, Di] bf16 or NULL: the first d_idx_rope columns of every head
 *     roped in place.
 * rope over a width d turns pair (x[2i], x[2i+1]) by pos * theta^(-2i/d).
 * Every value is computed in double and rounded once to bf16 (nearest,
 * ties to even).  Cache rows not named by pos are untouched. */
int oracle_cache_write(const uint16_t* kv_a, const float* norm_w, double eps,
                       const int64_t* pos, int64_t T, int64_t N,
                       uint16_t* kv_cache, const uint16_t* kI_new, uint16_t* kI_cache,
                       uint16_t* q, uint16_t* qI,
                       int32_t H, int32_t Dl, int32_t Dr, int32_t Hi, int32_t Di,
                       int32_t d_idx_rope, double theta);

/* Router selection per token (pipeline trace section 8a).
 *   logits [T, E] float, bias [E] float;
 *   p_e = sigmoid(logit_e) rounded once to float; s_e = p_e + bias_e (float);
 *   ids [T, k]: the k experts by (s desc, e asc), in that order;
 *   weights [T, k] double: p_e / max(sum of the k p_e, min_sum) * scale. */
int oracle_router_topk(const float* logits, const float* bias, int64_t T, int32_t E, int32_t k,
                       double scale, double min_sum, int32_t* ids, double* weights);

/* Value up-projection per head (pipeline trace section 6, kqv = v_mla . kqv):
 *   out_v[t, h, j] = bf16( sum_c bf16(o[t, h, c]) * wv[h, j, c] )
 *   o [T, H, Dl] float; wv [H, Dv, Dl] bf16; out_v [T, H, Dv] bf16. */
int oracle_value_up_proj(const float* o, const uint16_t* wv, int64_t T, int32_t H, int32_t Dl,
                         int32_t Dv, uint16_t* out_v);

/* Output projection for selected rows (rows == NULL: rows 0..nrows-1):
 *   y[r, n] = sum_k x[rows[r], k] * wo[n, k];  x [T, Kin], wo [Nout, Kin] bf16;
 *   y [nrows, Nout] double. */
int oracle_o_proj(const uint16_t* x, const uint16_t* wo, int64_t T, int32_t Kin, int32_t Nout,
                  const int64_t* rows, int64_t nrows, double* y);

/* Dense masked attention, non-absorbed form (exo PR #2539, Prefill section:
 * one 256-wide product per head under a boolean mask).
 * oracle_selection_mask: mask [L, W] uint32, bit j%32 of word j/32 set iff
 *   key j is in idx[i, :count[i]], 0 <= j < N and j <= q_start + i.
 * oracle_dense_masked_attn: q [L, H, Dn+Dr] bf16 (no-rope | rope);
 *   kvb [N, H, Dn+Dv] bf16 (no-rope key | value per head); kv [N, Dc] bf16
 *   whose columns rope_col .. rope_col+Dr-1 hold the shared rope key;
 *   out [nrows, H, Dv] double; a query with no masked-in key gets zeros. */
int oracle_selection_mask(const int32_t* idx, const int32_t* count, int64_t L, int32_t top_k,
                          int64_t N, int64_t q_start, int64_t W, uint32_t* mask);
int oracle_dense_masked_attn(const uint16_t* q, const uint16_t* kvb, const uint16_t* kv,
                             const uint32_t* mask, int64_t L, int64_t N, int32_t H, int32_t Dn,
                             int32_t Dr, int32_t Dv, int32_t Dc, int32_t rope_col, int64_t W,
                             double scale, const int64_t* rows, int64_t nrows, double* out,
                             int32_t nthreads);

/* The dense path's kv_b up-projection: kvb[j, h, c] = round(sum_d kv[j, d] *
 * w[h*(Dn+Dv) + c, d]) over the first Dl columns of each cache row (row
 * stride kv_cols); bf16 for c < Dn, and for c >= Dn too unless values_f16,
 * which rounds the value columns to fp16 instead (nearest even). */
int oracle_kv_b_proj(const uint16_t* kv, int32_t kv_cols, const uint16_t* w, int64_t N, int32_t H,
                     int32_t Dl, int32_t Dn, int32_t Dv, int32_t values_f16, uint16_t* kvb);

/* Query absorption: out[t, h, d] = round(sum_c q[t, h, c] * w[h*(Dn+Dv) + c, d])
 * for c < Dn, d < Dl (bf16, nearest even), and out[t, h, Dl + r] = q[t, h,
 * Dn + r] (the rope part). */
int oracle_q_absorb(const uint16_t* q, const uint16_t* w, int64_t T, int32_t H, int32_t Dn, int32_t Dr,
                    int32_t Dl, int32_t Dv, uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
