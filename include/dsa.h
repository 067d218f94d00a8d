/*
 * dsa.h - C ABI of the MI355X (gfx950) DeepSeek-sparse-attention core:
 * indexer scores -> top-k selection -> absorbed-MLA attention over the
 * selected latent rows, for one prefill chunk or one batched decode step.
 *
 * What is computed (the pages define it; section names, no line numbers):
 *  - exo PR #2539 "GLM-5.2/5.3 (glm_moe_dsa) attention and MoE speed-ups",
 *    Prefill section: a key's indexer score is the sum over the indexer heads
 *    of the head's weight times relu(q.k), summed in float32 with the causal
 *    mask applied; each query keeps its index_topk best causal keys, and a
 *    query with no more causal keys than that keeps every earlier key; the
 *    selected latent rows are gathered and attended with a float32 softmax.
 *    Decode section: single-token attention treats the heads as the rows of
 *    one product with the shared latent keys.
 *  - "GLM-5.2-Vision: llama.cpp vs vLLM line-by-line pipeline trace",
 *    section 6 (absorbed MLA): Q = [q_nope_absorbed | q_pe], K = [kv_cmpr |
 *    k_pe], V = kv_cmpr; the config line gives 64 heads, kv_lora_rank 512,
 *    qk_rope 64 and index_topk 2048.
 *
 * Readings taken where the pages are silent:
 *  - key j sits at position j and is visible to the query at position p iff
 *    j <= p; the indexer key is one Di-wide row per token shared by all
 *    indexer heads; w is per query and head; no other factor scales it;
 *  - equal scores go to the lower key index; a selection is listed in
 *    ascending key order, padded with -1, count = min(p + 1, top_k);
 *  - the softmax scale is an argument (GLM: 1/16 = 1/sqrt(192 + 64));
 *  - the output is the latent-space attention output in float32.
 *
 * Conventions for every call:
 *  - Pointers marked [dev] are device pointers owned by the caller, 16-byte
 *    aligned, dense row-major with the shapes given.  [host] pointers are
 *    read during the call only.  bf16 data is passed as uint16_t bits.
 *  - The library allocates nothing and keeps no state beyond a per-device
 *    architecture check and the device array dsa_decode_step_noalloc uses
 *    as its workspace.  Every call is asynchronous on `stream` (a
 *    hipStream_t; NULL = the default stream); it never synchronises and
 *    never reads device data on the host.
 *  - Arguments are validated before anything is enqueued; on any error
 *    nothing is enqueued and the status says why.  A failed launch returns
 *    DSA_ERR_HIP.  Non-finite inputs give undefined results.
 *  - Supported shapes: (n_heads, d_latent, d_rope, n_idx_heads, d_idx) =
 *    (64, 512, 64, 32, 128) (GLM-5.x) or (4, 64, 16, 4, 32) (tiny check
 *    shape); 1 <= top_k <= 2048; key counts up to DSA_MAX_SELECT_KEYS (262144)
 *    for selection.
 *    Others return DSA_ERR_UNSUPPORTED.  The device must be gfx950.
 *  - The value product runs with fp16 operands (probabilities and the first
 *    d_latent latent columns) and fp32 accumulation: latent values must lie
 *    within +-65504.  The score product runs in bf16 with fp32 accumulation.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size or position */
    DSA_ERR_UNSUPPORTED = -2,   /* shape, size or device this library does not handle */
    DSA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
    DSA_ERR_HIP = -4            /* a HIP runtime call or kernel launch failed */
} dsa_status;

typedef struct {
    int32_t n_heads;       /* H: query heads (GLM 64) */
    int32_t d_latent;      /* Dl: absorbed no-rope width = value width (GLM 512) */
    int32_t d_rope;        /* Dr: rope width (GLM 64); query/key width Dl + Dr */
    int32_t n_idx_heads;   /* Hi: indexer heads (GLM 32) */
    int32_t d_idx;         /* Di: indexer head width (128) */
    int32_t top_k;         /* keys kept per query (GLM index_topk 2048) */
    float softmax_scale;   /* multiplies q.k before the softmax (GLM 1/16) */
} dsa_shape;

/* Human-readable name of a status code (static string). */
const char* dsa_status_string(dsa_status status);

/* Indexer scores of L queries at positions q_start .. q_start+L-1 over keys
 * 0 .. N-1 (exo #2539, Prefill, float32 indexer):
 *   S[i, j] = sum_h w[i,h] * max(0, sum_d qI[i,h,d] * kI[j,d])   if j <= q_start+i
 *   S[i, j] = -infinity                                           otherwise.
 * qI [dev] [L, Hi, Di] bf16; kI [dev] [N, Di] bf16; w [dev] [L, Hi] fp32;
 * S [dev] [L, N] fp32 (written entirely).  Requires L >= 1, q_start >= 0,
 * q_start + L <= N.  Products are exact in fp32; sums accumulate in fp32. */
dsa_status dsa_indexer_scores(const dsa_shape* shape, const uint16_t* qI, const uint16_t* kI,
                              const float* w, int32_t L, int32_t N, int64_t q_start, float* S,
                              void* stream);

/* Top-k selection per query (exo #2539, Prefill: index_topk selection and
 * the every-earlier-key rule).  For the query at p = q_start + i:
 *   p + 1 <= top_k : idx[i] = 0, 1, .., p (S is not read);
 *   otherwise      : the top_k keys j <= p by (S desc, j asc), ascending.
 * S [dev] [L, N] fp32 (only j <= p read); idx [dev] [L, top_k] int32, padded
 * with -1; count [dev] [L] int32 = min(p + 1, top_k).  Requires
 * q_start + L <= N <= DSA_MAX_SELECT_KEYS.  Rows of up to 65536 keys take one
 * pass; longer rows take about (p + 1) / 63488 passes over pieces of the row. */
dsa_status dsa_topk_select(const dsa_shape* shape, const float* S, int32_t L, int32_t N,
                           int64_t q_start, int32_t* idx, int32_t* count, void* stream);

/* Absorbed-MLA attention of L queries over their selected latent rows
 * (pipeline trace section 6; exo #2539 Prefill sparse attention, Decode):
 *   s_t = softmax_scale * <q[i,h,:], kv[idx[i,t], :]>   for t < count[i]
 *   out[i,h,:] = sum_t softmax(s)_t * kv[idx[i,t], 0:Dl];  lse = log sum exp s.
 * q [dev] [L, H, Dl+Dr] bf16; kv [dev] [N, Dl+Dr] bf16; idx [dev] [L, top_k]
 * int32 in any order (entries outside [0, N) are skipped); count [dev] [L]
 * int32 (values above top_k are clamped); out [dev] [L, H, Dl] fp32;
 * lse [dev] [L, H] fp32 natural log, or NULL.  A row with no usable key
 * gets out = 0 and lse = -infinity.  Probabilities and latent values enter
 * the value product as fp16: requires |kv latent| <= 65504.  Rows are
 * addressed with 32-bit byte offsets: N * 2 * (Dl+Dr) must stay below 2^32
 * (DSA_ERR_UNSUPPORTED otherwise; 3.7 M rows at GLM shape). */
dsa_status dsa_sparse_mla_attn(const dsa_shape* shape, const uint16_t* q, const uint16_t* kv,
                               const int32_t* idx, const int32_t* count, int32_t L, int32_t N,
                               float* out, float* lse, void* stream);

/* Latent cache in the fp16-latent layout: kv16 has kv's shape [N, Dl+Dr];
 * its Dl latent columns hold kv's values converted bf16 -> fp16 (round to
 * nearest even) and its Dr rope columns are copied unchanged.  kv [dev],
 * kv16 [dev], caller-owned, 16-byte aligned, not overlapping.  The
 * conversion is exact for |v| in [2^-14, 65504]; smaller magnitudes become
 * fp16 subnormals (absolute error <= 2^-25), larger ones infinities, so the
 * fp16-latent path requires |v| <= 65504 (the value product already does,
 * see dsa_sparse_mla_attn). */
dsa_status dsa_latent_to_f16(const dsa_shape* shape, const uint16_t* kv, int32_t N, uint16_t* kv16,
                             void* stream);

/* dsa_sparse_mla_attn over an fp16-latent cache (dsa_latent_to_f16): the
 * same operation, arguments and errors, with kv16 in place of kv.  The
 * latent part of q is converted to fp16 inside the kernel (same range
 * condition as the cache), so the latent score products run on fp16
 * operands; the rope part stays bf16.  This is the kernel dsa_prefill_chunk
 * runs. */
dsa_status dsa_sparse_mla_attn_f16(const dsa_shape* shape, const uint16_t* q, const uint16_t* kv16,
                                   const int32_t* idx, const int32_t* count, int32_t L, int32_t N,
                                   float* out, float* lse, void* stream);

/* Workspace bytes dsa_prefill_chunk needs for this chunk geometry
 * (0 on invalid or unsupported arguments). */
size_t dsa_prefill_workspace_bytes(const dsa_shape* shape, int32_t L, int32_t N, int64_t q_start);

/* One prefill chunk end to end: L queries at q_start .. q_start+L-1 over
 * keys 0 .. N-1 with N = q_start + L (exo #2539, Prefill).  Queries with
 * p + 1 <= top_k skip the indexer and keep every earlier key; the rest are
 * scored, selected and attended over their top_k keys.
 * q [dev] [L,H,Dl+Dr], qI [dev] [L,Hi,Di] bf16; w [dev] [L,Hi] fp32;
 * kv [dev] [N,Dl+Dr], kI [dev] [N,Di] bf16; out [dev] [L,H,Dl] fp32;
 * idx_out [dev] [L,top_k] int32 or NULL; count_out [dev] [L] int32 or NULL;
 * ws [dev] of at least dsa_prefill_workspace_bytes() bytes.  The attention
 * runs on an fp16-latent copy of kv held in the workspace (see
 * dsa_latent_to_f16 for the range condition). */
dsa_status dsa_prefill_chunk(const dsa_shape* shape, const uint16_t* q, const uint16_t* qI,
                             const float* w, const uint16_t* kv, const uint16_t* kI, int32_t L,
                             int32_t N, int64_t q_start, float* out, int32_t* idx_out,
                             int32_t* count_out, void* ws, size_t ws_bytes, void* stream);

/* Largest batch dsa_decode_step accepts.  Batches of more than 128
 * sequences run as consecutive groups of 128 on the caller's stream (each
 * group a full set of launches); the workspace covers the largest group. */
#define DSA_MAX_DECODE_BATCH 16384
/* Most keys one selection reads (N of a prefill chunk, ctx of a decode
 * sequence). */
#define DSA_MAX_SELECT_KEYS 262144

/* Workspace bytes dsa_decode_step needs (0 on invalid arguments). */
size_t dsa_decode_workspace_bytes(const dsa_shape* shape, int32_t B, const int64_t* ctx);

/* One batched decode step (exo #2539, Decode): B sequences, one query each
 * at position ctx[b] - 1 over that sequence's ctx[b] cached keys.  Caches
 * are packed in sequence order: sequence b's rows start at sum(ctx[:b]).
 * ctx [host] [B], 1 <= ctx[b] <= DSA_MAX_SELECT_KEYS, B <= DSA_MAX_DECODE_BATCH;
 * q [dev] [B,H,Dl+Dr], qI [dev] [B,Hi,Di] bf16; w [dev] [B,Hi] fp32;
 * kv [dev] [sum ctx, Dl+Dr], kI [dev] [sum ctx, Di] bf16;
 * out [dev] [B,H,Dl] fp32; idx_out [dev] [B,top_k] int32 (key ids local to
 * the sequence) or NULL; count_out [dev] [B] or NULL; ws as above. */
dsa_status dsa_decode_step(const dsa_shape* shape, int32_t B, const int64_t* ctx,
                           const uint16_t* q, const uint16_t* qI, const float* w,
                           const uint16_t* kv, const uint16_t* kI, float* out, int32_t* idx_out,
                           int32_t* count_out, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the device-resident workspace dsa_decode_step_noalloc uses. */
#define DSA_DECODE_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/* dsa_decode_step without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same operation, arguments, results
 * and errors, with the workspace taken from a device array of
 * DSA_DECODE_STATIC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on, from its first call there until the process ends.  A step whose
 * workspace (dsa_decode_workspace_bytes) exceeds that size is rejected with
 * DSA_ERR_WORKSPACE before anything is enqueued (the 8-sequence 4k..64k
 * step needs about 17 MiB; 128 sequences of 65536 keys do not fit).  The
 * call itself allocates nothing; the first call on a device looks up the
 * array's device address once.  Every call on a GPU shares that GPU's
 * array, and every buffer in it is written before it is read, so nothing
 * from an earlier call leaks into a later one; calls that overlap on one
 * GPU (concurrent streams, or threads) race on it and must be serialised
 * by the caller. */
dsa_status dsa_decode_step_noalloc(const dsa_shape* shape, int32_t B, const int64_t* ctx,
                                   const uint16_t* q, const uint16_t* qI, const float* w,
                                   const uint16_t* kv, const uint16_t* kI, float* out, int32_t* idx_out,
                                   int32_t* count_out, void* stream);

/* Upstream cache write of T new tokens ("GLM-5.2-Vision: llama.cpp vs vLLM
 * line-by-line pipeline trace", section 4, KV compression path: kv_cmpr and
 * k_pe are split from the kv_a projection output, q_pe and k_pe are roped,
 * kv_cmpr is RMS-normalised after the split; section 5: the rope is the NORM
 * flavour, adjacent pairs, and the indexer rope is NORM too).  For token t
 * at position p = pos[t]:
 *   kv[p, 0:Dl]     = kv_a[t, 0:Dl] / sqrt(mean(kv_a[t, 0:Dl]^2) + eps) * norm_w
 *   kv[p, Dl:Dl+Dr] = rope(kv_a[t, Dl:Dl+Dr], p)
 *   kI[p, :]        = kI_new[t, :] with columns 0 .. d_idx_rope-1 roped
 *   q[t, h, Dl:Dl+Dr] and qI[t, hi, 0:d_idx_rope] roped in place
 * where rope over a width d turns the pair (x[2i], x[2i+1]) by the angle
 * p * rope_theta^(-2i/d).  rope_theta, eps and d_idx_rope are not on the
 * pages; they are arguments.
 * kv_a [dev] [T, Dl+Dr] bf16; norm_w [dev] [Dl] fp32; pos [dev] [T] int32;
 * kv [dev] [N, Dl+Dr] bf16 cache; kI_new [dev] [T, Di] and kI [dev] [N, Di]
 * bf16 (both NULL: no indexer key is written); q [dev] [T, H, Dl+Dr] bf16 or
 * NULL; qI [dev] [T, Hi, Di] bf16 or NULL.  Cache rows are written only for
 * tokens with 0 <= pos < N (the query rope uses pos as given); positions
 * must be distinct (two tokens writing one row race), and kv_a / kI_new must
 * not overlap the rows written.  Results are computed in double precision
 * and rounded once to bf16 (nearest, ties to even), for values in the normal
 * bf16 range.  Requires T >= 0 (0: nothing is enqueued), N >= 1,
 * rope_theta > 0, eps >= 0, 0 <= d_idx_rope <= Di; d_idx_rope must be a
 * multiple of 8 (DSA_ERR_UNSUPPORTED otherwise).  kv_a, kv, kI_new, kI, q,
 * qI 16-byte aligned; norm_w and pos 4-byte aligned. */
dsa_status dsa_cache_write(const dsa_shape* shape, const uint16_t* kv_a, const float* norm_w, float eps,
                           const int32_t* pos, int32_t T, int32_t N, uint16_t* kv, const uint16_t* kI_new,
                           uint16_t* kI, uint16_t* q, uint16_t* qI, int32_t d_idx_rope, float rope_theta,
                           void* stream);

/* MoE router selection for T tokens ("GLM-5.2-Vision: llama.cpp vs vLLM
 * line-by-line pipeline trace", section 8a, Gating; exo PR #2539, router
 * selection in one kernel).  Per token, with p_e = sigmoid(logits[t, e]):
 *   s_e = p_e + bias[e]                        (the bias serves the choice only)
 *   ids[t, :] = the k experts by (s desc, e asc), in that order
 *   weights[t, j] = p_ids[j] / max(sum_j p_ids[j], 6.1e-5) * routed_scale
 * (GLM: 256 experts, k = 8, routed_scale 2.5, one expert group).  Readings:
 * p_e is the exact sigmoid rounded once to float; s_e is a float sum; equal
 * scores go to the lower expert index.  Weights are formed in double and
 * rounded to float.
 * logits [dev] [T, n_experts] fp32 (16-byte aligned); bias [dev]
 * [n_experts] fp32; ids [dev] [T, k] int32; weights [dev] [T, k] fp32.
 * Requires T >= 0 (0: nothing is enqueued), 1 <= k <= n_experts, a finite
 * routed_scale; n_experts in {64, 128, 256, 512, 1024} and k <= 32
 * (DSA_ERR_UNSUPPORTED otherwise).  Non-finite logits or biases give
 * undefined results. */
dsa_status dsa_router_topk(const float* logits, const float* bias, int32_t T, int32_t n_experts, int32_t k,
                           float routed_scale, int32_t* ids, float* weights, void* stream);

/* Value up-projection per head ("GLM-5.2-Vision: llama.cpp vs vLLM
 * line-by-line pipeline trace", section 6, build_attn: the latent-space
 * attention output is decompressed per head with wv_b, kqv = v_mla . kqv;
 * the config line gives v_head_dim 256):
 *   out_v[t, h, j] = bf16( sum_c bf16(o[t, h, c]) * wv[h, j, c] )
 * o [dev] [T, H, Dl] fp32 (the attention output); wv [dev] [H, d_v, Dl]
 * bf16 (stored [out, in]); out_v [dev] [T, H, d_v] bf16.  The products take
 * bf16 operands (o is rounded to nearest-even once) and accumulate in fp32;
 * the result is rounded once to bf16.  Requires T >= 0 (0: nothing is
 * enqueued); d_v must be 256 and Dl a multiple of 64 (DSA_ERR_UNSUPPORTED
 * otherwise); all pointers 16-byte aligned. */
dsa_status dsa_value_up_proj(const dsa_shape* shape, const float* o, const uint16_t* wv, int32_t T, int32_t d_v,
                             uint16_t* out_v, void* stream);

/* Output projection (pipeline trace section 6: the up-projected heads,
 * flattened, times wo; config line: hidden 6144):
 *   y[t, n] = sum_k x[t, k] * wo[n, k]
 * x [dev] [T, k_in] bf16 (e.g. out_v viewed as [T, H * d_v]); wo [dev]
 * [n_out, k_in] bf16 (stored [out, in]); y [dev] [T, n_out] fp32.  bf16
 * operands, fp32 accumulation.  Requires T >= 0 (0: nothing is enqueued);
 * k_in a multiple of 64 and n_out a multiple of 192 (DSA_ERR_UNSUPPORTED
 * otherwise); all pointers 16-byte aligned. */
dsa_status dsa_o_proj(const uint16_t* x, const uint16_t* wo, int32_t T, int32_t k_in, int32_t n_out, float* y,
                      void* stream);

/* Selection mask for the dense path (exo PR #2539, Prefill section: below
 * 8192 keys the attention runs dense under a boolean mask; the mask is the
 * query's DSA selection, which for a query with no more causal keys than
 * top_k is every earlier key):
 *   mask[i, w] bit b set  iff  key j = 32 w + b is among idx[i, :count[i]],
 *                              0 <= j < N and j <= q_start + i.
 * idx [dev] [L, top_k] int32 (as dsa_topk_select writes it; other entries are
 * ignored, a key listed twice is set once); count [dev] [L] int32 (clamped to
 * [0, top_k]); mask [dev] [L, mask_words] uint32, fully written (bits at or
 * past N are 0).  Requires L >= 0 (0: nothing is enqueued), top_k >= 1,
 * N >= 1, q_start >= 0, mask_words >= 2 * ceil(N / 64) (whole 64-key tiles);
 * mask_words <= 16384 (DSA_ERR_UNSUPPORTED otherwise). */
dsa_status dsa_selection_mask(const int32_t* idx, const int32_t* count, int32_t L, int32_t top_k, int32_t N,
                              int32_t q_start, int32_t mask_words, uint32_t* mask, void* stream);

/* Dense masked attention, non-absorbed form (exo PR #2539, Prefill section,
 * dense attention in one product: each head's no-rope and rope dimensions
 * are scored in one product under a boolean mask; widths from the config
 * line of "GLM-5.2-Vision: llama.cpp vs vLLM line-by-line pipeline trace":
 * qk_nope 192, qk_rope 64, v_head_dim 256; its section 4 splits the kv_b
 * output per head into the no-rope key and the value, and k_pe is shared):
 *   s[i,h,j] = scale * ( q[i,h,:Dn] . kvb[j,h,:Dn] + q[i,h,Dn:] . kv[j, rope_col : rope_col+Dr] )
 *   out[i,h,:] = sum over masked-in j of softmax_j(s) * kvb[j,h,Dn:Dn+Dv]
 * for the query at position q_start + i; keys after it are never used.
 * q [dev] [L, H, Dn+Dr] bf16; kvb [dev] [N, H, Dn+Dv] bf16 (the kv_b
 * projection of the latent rows); kv [dev] [N, kv_cols] bf16 (cache rows,
 * rope key at rope_col); mask [dev] [L, mask_words] as dsa_selection_mask
 * writes it; out [dev] [L, H, Dv] fp32; a query with no masked-in key gets
 * zeros.  bf16 score products with fp32 sums, fp32 softmax, probabilities
 * rounded to fp16 and values converted to fp16 for the value product (|v|
 * must stay below 65504).  (Dn, Dr, Dv) must be (192, 64, 256) or
 * (64, 64, 64) (DSA_ERR_UNSUPPORTED otherwise); q, kvb, kv, out 16-byte
 * aligned, mask 4-byte aligned; kv_cols and rope_col multiples of 8;
 * mask_words >= 2 * ceil(N / 64); scale finite and > 0; L >= 0 (0: nothing
 * is enqueued), N >= 1, H >= 1. */
dsa_status dsa_dense_masked_attn(const uint16_t* q, const uint16_t* kvb, const uint16_t* kv, int32_t kv_cols,
                                 int32_t rope_col, const uint32_t* mask, int32_t mask_words, int32_t L,
                                 int32_t N, int32_t q_start, int32_t H, int32_t d_nope, int32_t d_rope,
                                 int32_t d_v, float scale, float* out, void* stream);

/* dsa_dense_masked_attn with the values in the fp16 form vt instead of the
 * bf16 value columns of kvb (whose no-rope key columns are still read):
 *   vt [dev] [H, d_v, Np] fp16, Np = N rounded up to a multiple of 64,
 *   positions N..Np-1 zero; feature row (h, f) holds key k at position
 *   32 * (k / 32) + vt_pos(k % 32), vt_pos(x) = 8 * ((x % 16) / 4) +
 *   4 * (x / 16) + x % 4 (the order in which the kernel's probability
 *   fragments list a 32-key step's keys, so one 16-byte read is one matrix
 *   operand).  dsa_values_to_f16 or dsa_kv_b_proj writes it.  Same
 *   arguments, results and requirements otherwise; vt must be non-null and
 *   16-byte aligned. */
dsa_status dsa_dense_masked_attn_f16(const uint16_t* q, const uint16_t* kvb, const uint16_t* vt, const uint16_t* kv,
                                     int32_t kv_cols, int32_t rope_col, const uint32_t* mask, int32_t mask_words,
                                     int32_t L, int32_t N, int32_t q_start, int32_t H, int32_t d_nope,
                                     int32_t d_rope, int32_t d_v, float scale, float* out, void* stream);

/* The value columns of kvb [dev] [N, H, d_nope + d_v] (bf16) into the fp16
 * form vt [dev] [H, d_v, Np] that dsa_dense_masked_attn_f16 reads (layout
 * there), rounded to nearest even (exact for |v| in [2^-14, 65504]; smaller
 * magnitudes become fp16 subnormals, larger ones infinities), positions
 * N..Np-1 zero.  Requires kvb and vt 16-byte aligned and not overlapping,
 * N >= 0 (0: nothing is enqueued), H >= 1, d_nope a multiple of 8; d_v 64
 * or 256 and H <= 65535 (DSA_ERR_UNSUPPORTED otherwise). */
dsa_status dsa_values_to_f16(const uint16_t* kvb, int32_t N, int32_t H, int32_t d_nope, int32_t d_v, uint16_t* vt,
                             void* stream);

/* kv_b up-projection of the latent rows for the dense path ("GLM-5.2-Vision:
 * llama.cpp vs vLLM line-by-line pipeline trace", section 4: the kv_b
 * projection of the normalised latent gives each head's no-rope key and
 * value; config line: qk_nope 192, v_head_dim 256):
 *   kvb[j, h, c] = sum_d kv[j, d] * wkvb[h * (d_nope + d_v) + c, d],  d < d_latent
 * kv [dev] [N, kv_cols] bf16 (the cache rows; the latent is their first
 * d_latent columns); wkvb [dev] [H * (d_nope + d_v), d_latent] bf16 (stored
 * [out, in]); kvb [dev] [N, H, d_nope + d_v] receives the bf16 no-rope keys
 * and, when vt is NULL, the bf16 values; with vt non-null the values go to
 * vt [dev] [H, d_v, Np] in fp16 instead (the form dsa_dense_masked_attn_f16
 * reads, layout there; magnitudes from 65520 up become infinities;
 * positions N..Np-1 written as zeros) and kvb's value columns are left
 * alone.  bf16 products, fp32 sums, each result rounded once (nearest
 * even).  Requires N >= 0 (0: nothing is enqueued), H >= 1, pointers 16-byte
 * aligned, kv_cols a multiple of 8; d_latent a multiple of 64 and
 * H * (d_nope + d_v) a multiple of 256 (DSA_ERR_UNSUPPORTED otherwise). */
dsa_status dsa_kv_b_proj(const uint16_t* kv, int32_t kv_cols, const uint16_t* wkvb, int32_t N, int32_t H,
                         int32_t d_latent, int32_t d_nope, int32_t d_v, uint16_t* kvb, uint16_t* vt,
                         void* stream);

/* Query absorption ("GLM-5.2-Vision: llama.cpp vs vLLM line-by-line
 * pipeline trace", section 6: q_nope_absorbed, the query the absorbed-MLA
 * attention scores the shared latent rows with):
 *   q_abs[t, h, d]      = sum_c q[t, h, c] * wkvb[h * (d_nope + d_v) + c, d],  c < d_nope, d < d_latent
 *   q_abs[t, h, d_latent + r] = q[t, h, d_nope + r],  r < d_rope (the rope part, copied)
 * so that <q_abs[t, h, :d_latent], kv row> equals the no-rope query's score
 * against that row's up-projected key (dsa_kv_b_proj) before rounding.
 * q [dev] [T, H, d_nope + d_rope] bf16; wk_t [dev] [H, d_latent, d_nope]
 * bf16, the key block of the kv_b weight transposed per head (wk_t[h, d, c]
 * = wkvb[h * (d_nope + d_v) + c, d]; dsa_absorb_weight writes it once per
 * weight); q_abs [dev] [T, H, d_latent + d_rope] bf16, the query layout of
 * dsa_sparse_mla_attn.  bf16 products, fp32 sums, each result rounded once
 * (nearest even).  Requires pointers 16-byte aligned, T >= 0 (0: nothing is
 * enqueued), H >= 1; d_nope a multiple of 64, d_latent a multiple of 256,
 * d_rope a multiple of 8 and T * H * (d_nope + d_rope) * 2 < 2^32
 * (DSA_ERR_UNSUPPORTED otherwise). */
dsa_status dsa_q_absorb(const uint16_t* q, const uint16_t* wk_t, int32_t T, int32_t H, int32_t d_nope,
                        int32_t d_rope, int32_t d_latent, uint16_t* q_abs, void* stream);

/* The weight dsa_q_absorb reads: wk_t [dev] [H, d_latent, d_nope] bf16,
 * wk_t[h, d, c] = wkvb[h * (d_nope + d_v) + c, d], from the kv_b weight
 * wkvb [dev] [H * (d_nope + d_v), d_latent] bf16 (stored [out, in], as
 * dsa_kv_b_proj reads it).  Not overlapping; H, d_nope, d_latent >= 1,
 * d_v >= 0. */
dsa_status dsa_absorb_weight(const uint16_t* wkvb, int32_t H, int32_t d_nope, int32_t d_v, int32_t d_latent,
                             uint16_t* wk_t, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
