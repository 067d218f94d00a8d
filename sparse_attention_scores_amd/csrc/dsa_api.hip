// dsa_api.hip - the C ABI declared in include/dsa.h: argument validation,
// workspace layout, launch geometry and stream ordering.  All checks run
// before anything is enqueued; nothing here reads device memory.
#include "../../include/dsa.h"
#include "dsa_kernels.h"

#include <cmath>

#include <math.h>
#include <string.h>

#include <mutex>

static_assert(dsa::kMaxSelectKeys == DSA_MAX_SELECT_KEYS, "header limit matches the kernels'");

namespace {

using dsa::SeqMeta;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 0 = GLM-5.x (64, 512, 64, 32, 128); 1 = tiny check shape (4, 64, 16, 4, 32); -1 otherwise
int shape_id(const dsa_shape* s) {
    if (!s) return -1;
    if (s->n_heads == 64 && s->d_latent == 512 && s->d_rope == 64 && s->n_idx_heads == 32 && s->d_idx == 128)
        return 0;
    if (s->n_heads == 4 && s->d_latent == 64 && s->d_rope == 16 && s->n_idx_heads == 4 && s->d_idx == 32)
        return 1;
    return -1;
}

dsa_status check_shape(const dsa_shape* s) {
    if (!s) return DSA_ERR_INVALID_ARG;
    if (s->n_heads <= 0 || s->d_latent <= 0 || s->d_rope < 0 || s->n_idx_heads <= 0 || s->d_idx <= 0 ||
        s->top_k <= 0 || !isfinite(s->softmax_scale))
        return DSA_ERR_INVALID_ARG;
    if (shape_id(s) < 0 || s->top_k > dsa::kMaxTopK) return DSA_ERR_UNSUPPORTED;
    return DSA_OK;
}

// The kernels are built for gfx950 only; refuse any other current device.
dsa_status check_device() {
    static std::mutex mu;
    static int known[64];   // 0 unknown, 1 gfx950, 2 other
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_HIP;
    if (dev < 0 || dev >= 64) return DSA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (known[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DSA_ERR_HIP;
        known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    }
    return known[dev] == 1 ? DSA_OK : DSA_ERR_UNSUPPORTED;
}

dsa_status launched(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_HIP; }

float scale_log2(const dsa_shape* s) { return s->softmax_scale * 1.4426950408889634f; }

// first query row of a chunk that is scored (p + 1 > top_k)
int32_t first_sparse_row(int32_t L, int64_t q_start, int32_t top_k) {
    int64_t i0 = (int64_t)top_k - q_start;
    if (i0 < 0) i0 = 0;
    if (i0 > L) i0 = L;
    return (int32_t)i0;
}

int64_t padded_row(int64_t n) { return (n + 63) / 64 * 64; }
// The attention gathers address a row through a 32-bit byte offset.
bool attn_keys_ok(const dsa_shape* s, int64_t N) {
    return N * 2 * (int64_t)(s->d_latent + s->d_rope) + 2 * (int64_t)(s->d_latent + s->d_rope) <= 0xFFFFFFFFll;
}

struct PrefillLayout {
    size_t s_off, idx_off, cnt_off, kv16_off, total;
    int32_t row0;
    int64_t ldS;
};

PrefillLayout prefill_layout(const dsa_shape* s, int32_t L, int32_t N, int64_t q_start) {
    PrefillLayout p;
    p.row0 = first_sparse_row(L, q_start, s->top_k);
    p.ldS = padded_row(N);
    p.s_off = 0;
    p.idx_off = align_up((size_t)(L - p.row0) * (size_t)p.ldS * sizeof(float));
    p.cnt_off = p.idx_off + align_up((size_t)L * s->top_k * sizeof(int32_t));
    p.kv16_off = p.cnt_off + align_up((size_t)L * sizeof(int32_t));
    p.total = p.kv16_off + align_up((size_t)N * (s->d_latent + s->d_rope) * sizeof(uint16_t));
    return p;
}

struct DecodeLayout {
    SeqMeta idx_meta;    // blocks of the indexer kernel
    SeqMeta attn_meta;   // blocks (chunks) of the attention kernel
    SeqMeta topk_meta;   // segment blocks of the top-k
    int idx_blocks, attn_items, chunk, n_max;
    size_t s_off, idx_off, cnt_off, po_off, pml_off, cand_off, total;
};

// Chunk of selected keys per attention block: about 128 blocks per step (a
// block's fixed cost, its query fragments and partial output, outweighs
// filling every CU with shorter chunks), at least one 32-key tile each.
int decode_chunk(const dsa_shape* s, int32_t B, const int64_t* ctx) {
    int64_t sel = 0;
    for (int b = 0; b < B; ++b) sel += ctx[b] < s->top_k ? ctx[b] : s->top_k;
    int64_t c = (sel + 127) / 128;
    c = (c + 31) / 32 * 32;
    if (c < 32) c = 32;
    if (c > s->top_k) c = (s->top_k + 31) / 32 * 32;
    return (int)c;
}

dsa_status decode_layout(const dsa_shape* s, int32_t B, const int64_t* ctx, DecodeLayout& d) {
    if (B <= 0 || !ctx) return DSA_ERR_INVALID_ARG;
    if (B > dsa::kMaxBatch) return DSA_ERR_UNSUPPORTED;
    memset(&d, 0, sizeof d);
    d.chunk = decode_chunk(s, B, ctx);
    const int kpb = dsa::indexer_decode_keys_per_block();
    int64_t koff = 0, soff = 0;
    int iblk = 0, items = 0, tblk = 0;
    d.n_max = 1;
    for (int b = 0; b < B; ++b) {
        if (ctx[b] <= 0) return DSA_ERR_INVALID_ARG;
        if (ctx[b] > dsa::kMaxSelectKeys) return DSA_ERR_UNSUPPORTED;
        const int c = (int)ctx[b];
        d.idx_meta.key_off[b] = d.attn_meta.key_off[b] = koff;
        d.idx_meta.s_off[b] = d.attn_meta.s_off[b] = soff;
        d.idx_meta.ctx[b] = d.attn_meta.ctx[b] = c;
        d.idx_meta.blk0[b] = iblk;
        d.attn_meta.blk0[b] = items;
        d.topk_meta.key_off[b] = koff;
        d.topk_meta.s_off[b] = soff;
        d.topk_meta.ctx[b] = c;
        d.topk_meta.blk0[b] = tblk;
        tblk += dsa::topk_decode_segments(c, s->top_k);
        // a sequence within top_k keeps every key: no scores needed
        if (c > s->top_k) iblk += (c + kpb - 1) / kpb;
        const int cnt = c < s->top_k ? c : s->top_k;
        items += (cnt + d.chunk - 1) / d.chunk;
        if (c > d.n_max) d.n_max = c;
        koff += c;
        soff += padded_row(c);
    }
    d.idx_meta.B = d.attn_meta.B = B;
    d.idx_meta.key_off[B] = d.attn_meta.key_off[B] = koff;
    d.idx_meta.s_off[B] = d.attn_meta.s_off[B] = soff;
    d.idx_meta.blk0[B] = iblk;
    d.attn_meta.blk0[B] = items;
    d.topk_meta.B = B;
    d.topk_meta.key_off[B] = koff;
    d.topk_meta.s_off[B] = soff;
    d.topk_meta.blk0[B] = tblk;
    d.idx_blocks = iblk;
    d.attn_items = items;
    d.s_off = 0;
    d.idx_off = align_up((size_t)soff * sizeof(float));
    d.cnt_off = d.idx_off + align_up((size_t)B * s->top_k * sizeof(int32_t));
    d.po_off = d.cnt_off + align_up((size_t)B * sizeof(int32_t));
    d.pml_off = d.po_off + align_up((size_t)items * s->n_heads * s->d_latent * sizeof(float));
    d.cand_off = d.pml_off + align_up((size_t)items * s->n_heads * 2 * sizeof(float));
    d.total = d.cand_off + align_up(dsa::topk_decode_work_bytes(B, tblk, s->top_k));
    return DSA_OK;
}

// Batches of more than kMaxBatch sequences (the most one launch's kernel
// arguments describe) run as consecutive groups of kMaxBatch sequences on
// the caller's stream, each group over the whole workspace (stream order
// keeps them apart).  f(b0, n, key_row0) runs for each group in order.
template <typename F>
dsa_status for_each_group(int32_t B, const int64_t* ctx, F&& f) {
    int64_t k0 = 0;
    for (int32_t b0 = 0; b0 < B; b0 += dsa::kMaxBatch) {
        const int32_t n = B - b0 < dsa::kMaxBatch ? B - b0 : dsa::kMaxBatch;
        const dsa_status st = f(b0, n, k0);
        if (st) return st;
        for (int32_t b = b0; b < b0 + n; ++b) k0 += ctx[b];
    }
    return DSA_OK;
}

// Workspace bytes of a batch: the largest group's layout (no HIP call).
dsa_status decode_need(const dsa_shape* s, int32_t B, const int64_t* ctx, size_t& need) {
    if (B <= 0 || !ctx) return DSA_ERR_INVALID_ARG;
    if (B > DSA_MAX_DECODE_BATCH) return DSA_ERR_UNSUPPORTED;
    static thread_local DecodeLayout d;
    need = 0;
    return for_each_group(B, ctx, [&](int32_t b0, int32_t n, int64_t) {
        const dsa_status st = decode_layout(s, n, ctx + b0, d);
        if (!st && d.total > need) need = d.total;
        return st;
    });
}

// Argument checks and workspace size shared by both decode entry points (no
// HIP call, nothing enqueued).
dsa_status decode_check(const dsa_shape* shape, int32_t B, const int64_t* ctx, const uint16_t* q,
                        const uint16_t* qI, const float* w, const uint16_t* kv, const uint16_t* kI,
                        const float* out, const int32_t* idx_out, const int32_t* count_out, size_t& need) {
    dsa_status st = check_shape(shape);
    if (st) return st;
    if (!q || !qI || !w || !kv || !kI || !out)
        return DSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(qI) || !aligned16(w) || !aligned16(kv) || !aligned16(kI) ||
        !aligned16(out) || (idx_out && !aligned16(idx_out)) || (count_out && !aligned16(count_out)))
        return DSA_ERR_INVALID_ARG;
    return decode_need(shape, B, ctx, need);
}

// The decode kernels over a workspace at `base` laid out as d says.
dsa_status decode_run(const dsa_shape* shape, const uint16_t* q, const uint16_t* qI, const float* w,
                      const uint16_t* kv, const uint16_t* kI, float* out, int32_t* idx_out, int32_t* count_out,
                      const DecodeLayout& d, char* base, hipStream_t s) {
    dsa_status st;
    const int sid = shape_id(shape);
    float* S = reinterpret_cast<float*>(base + d.s_off);
    int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + d.idx_off);
    int32_t* cnt = count_out ? count_out : reinterpret_cast<int32_t*>(base + d.cnt_off);
    if ((st = launched(dsa::launch_indexer_decode(sid, qI, kI, w, S, d.idx_meta, d.idx_blocks, s)))) return st;
    if ((st = launched(dsa::launch_topk_decode(S, d.topk_meta, shape->top_k, idx, cnt, base + d.cand_off, s))))
        return st;
    const dsa::DecWork dw = dsa::topk_decode_work(base + d.cand_off, d.topk_meta.B, d.topk_meta.blk0[d.topk_meta.B],
                                                  shape->top_k);
    dsa::AttnSplitArgs aa{q, kv, idx, cnt, dw, shape->top_k, d.chunk, scale_log2(shape),
                          reinterpret_cast<float*>(base + d.po_off), reinterpret_cast<float*>(base + d.pml_off),
                          out};
    return launched(dsa::launch_attention_split(sid, aa, d.attn_meta, d.attn_items, s));
}


// Every group of a checked batch over the workspace at `base`.  Each group's
// operands start at its first sequence (row b0 of q, qI, w, out, idx and
// count; cache row key_row0 of kv and kI).  Every group's tensor offsets stay
// 16-byte aligned: a sequence's rows and a cache row are whole multiples of
// 16 bytes at the supported shapes.
dsa_status decode_groups(const dsa_shape* s, int32_t B, const int64_t* ctx, const uint16_t* q,
                         const uint16_t* qI, const float* w, const uint16_t* kv, const uint16_t* kI, float* out,
                         int32_t* idx_out, int32_t* count_out, char* base, hipStream_t stream) {
    static thread_local DecodeLayout d;
    const int64_t dqk = (int64_t)s->d_latent + s->d_rope, dq = (int64_t)s->n_idx_heads * s->d_idx;
    return for_each_group(B, ctx, [&](int32_t b0, int32_t n, int64_t k0) {
        dsa_status st = decode_layout(s, n, ctx + b0, d);
        if (st) return st;
        return decode_run(s, q + b0 * s->n_heads * dqk, qI + b0 * dq, w + (int64_t)b0 * s->n_idx_heads,
                          kv + k0 * dqk, kI + k0 * s->d_idx, out + (int64_t)b0 * s->n_heads * s->d_latent,
                          idx_out ? idx_out + (int64_t)b0 * s->top_k : nullptr, count_out ? count_out + b0 : nullptr,
                          d, base, stream);
    });
}

}  // namespace

// Workspace of dsa_decode_step_noalloc: one array per device, resident from
// the library's first use on that device until the process ends.  Host code
// never passes the array's name to a kernel or a copy: the name is a
// host-side stand-in, and the device address comes from
// hipGetSymbolAddress (static_scratch below).
__device__ __attribute__((aligned(256))) unsigned char scratch[DSA_DECODE_STATIC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
dsa_status static_scratch(void** ptr) {
    static std::mutex mu;
    static void* addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_HIP;
    if (dev < 0 || dev >= 64) return DSA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DSA_ERR_HIP;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status status) {
    switch (status) {
        case DSA_OK: return "DSA_OK";
        case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG: null or misaligned pointer, or bad size/position";
        case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED: shape, size or device not handled by this library";
        case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE: workspace missing or too small";
        case DSA_ERR_HIP: return "DSA_ERR_HIP: a HIP call or kernel launch failed";
    }
    return "unknown dsa_status";
}

dsa_status dsa_indexer_scores(const dsa_shape* shape, const uint16_t* qI, const uint16_t* kI,
                              const float* w, int32_t L, int32_t N, int64_t q_start, float* S,
                              void* stream) {
    dsa_status st = check_shape(shape);
    if (st) return st;
    if (!qI || !kI || !w || !S || !aligned16(qI) || !aligned16(kI) || !aligned16(w) || !aligned16(S))
        return DSA_ERR_INVALID_ARG;
    if (L <= 0 || N <= 0 || q_start < 0 || q_start + L > N) return DSA_ERR_INVALID_ARG;
    if ((st = check_device())) return st;
    dsa::IndexerArgs a{qI, kI, w, S, N, L, N, q_start, 1};
    return launched(dsa::launch_indexer_prefill(shape_id(shape), a, (hipStream_t)stream));
}

dsa_status dsa_topk_select(const dsa_shape* shape, const float* S, int32_t L, int32_t N,
                           int64_t q_start, int32_t* idx, int32_t* count, void* stream) {
    dsa_status st = check_shape(shape);
    if (st) return st;
    if (!S || !idx || !count || !aligned16(S) || !aligned16(idx) || !aligned16(count))
        return DSA_ERR_INVALID_ARG;
    if (L <= 0 || N <= 0 || q_start < 0 || q_start + L > N) return DSA_ERR_INVALID_ARG;
    if (N > dsa::kMaxSelectKeys) return DSA_ERR_UNSUPPORTED;
    if ((st = check_device())) return st;
    dsa::TopkArgs a{S, N, 0, L, q_start, shape->top_k, idx, count};
    return launched(dsa::launch_topk_prefill(a, (int)(q_start + L), (hipStream_t)stream));
}

dsa_status dsa_sparse_mla_attn(const dsa_shape* shape, const uint16_t* q, const uint16_t* kv,
                               const int32_t* idx, const int32_t* count, int32_t L, int32_t N,
                               float* out, float* lse, void* stream) {
    dsa_status st = check_shape(shape);
    if (st) return st;
    if (!q || !kv || !idx || !count || !out || !aligned16(q) || !aligned16(kv) || !aligned16(out) ||
        (lse && !aligned16(lse)))
        return DSA_ERR_INVALID_ARG;
    if (L <= 0 || N <= 0) return DSA_ERR_INVALID_ARG;
    if (!attn_keys_ok(shape, N)) return DSA_ERR_UNSUPPORTED;
    if ((st = check_device())) return st;
    dsa::AttnArgs a{q, kv, idx, count, L, N, shape->top_k, scale_log2(shape), out, lse};
    return launched(dsa::launch_attention(shape_id(shape), a, false, (hipStream_t)stream));
}

dsa_status dsa_latent_to_f16(const dsa_shape* shape, const uint16_t* kv, int32_t N, uint16_t* kv16,
                             void* stream) {
    dsa_status st = check_shape(shape);
    if (st) return st;
    if (!kv || !kv16 || !aligned16(kv) || !aligned16(kv16) || N <= 0) return DSA_ERR_INVALID_ARG;
    if ((st = check_device())) return st;
    return launched(dsa::launch_latent_to_f16(shape_id(shape), kv, kv16, N, (hipStream_t)stream));
}

dsa_status dsa_cache_write(const dsa_shape* shape, const uint16_t* kv_a, const float* norm_w, float eps,
                           const int32_t* pos, int32_t T, int32_t N, uint16_t* kv, const uint16_t* kI_new,
                           uint16_t* kI, uint16_t* q, uint16_t* qI, int32_t d_idx_rope, float rope_theta,
                           void* stream) {
    dsa_status st = check_shape(shape);
    if (st) return st;
    if (!kv_a || !norm_w || !pos || !kv || !aligned16(kv_a) || !aligned16(kv) ||
        (reinterpret_cast<uintptr_t>(norm_w) & 3u) || (reinterpret_cast<uintptr_t>(pos) & 3u))
        return DSA_ERR_INVALID_ARG;
    if ((!kI_new) != (!kI) || (kI_new && (!aligned16(kI_new) || !aligned16(kI))) || (q && !aligned16(q)) ||
        (qI && !aligned16(qI)))
        return DSA_ERR_INVALID_ARG;
    if (T < 0 || N <= 0 || d_idx_rope < 0 || d_idx_rope > shape->d_idx || !(rope_theta > 0.f) ||
        !isfinite(rope_theta) || !(eps >= 0.f) || !isfinite(eps))
        return DSA_ERR_INVALID_ARG;
    if (d_idx_rope % 8 != 0) return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    if ((st = check_device())) return st;
    dsa::CacheWriteArgs a{kv_a, norm_w, pos, kI_new, kv, kI, q, qI, T, N, d_idx_rope, eps, rope_theta};
    return launched(dsa::launch_cache_write(shape_id(shape), a, (hipStream_t)stream));
}

dsa_status dsa_router_topk(const float* logits, const float* bias, int32_t T, int32_t n_experts, int32_t k,
                           float routed_scale, int32_t* ids, float* weights, void* stream) {
    if (!logits || !bias || !ids || !weights || !aligned16(logits) || (reinterpret_cast<uintptr_t>(bias) & 3u) ||
        (reinterpret_cast<uintptr_t>(ids) & 3u) || (reinterpret_cast<uintptr_t>(weights) & 3u))
        return DSA_ERR_INVALID_ARG;
    if (T < 0 || n_experts <= 0 || k <= 0 || k > n_experts || !isfinite(routed_scale)) return DSA_ERR_INVALID_ARG;
    if ((n_experts != 64 && n_experts != 128 && n_experts != 256 && n_experts != 512 && n_experts != 1024) ||
        k > 32)
        return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    dsa_status st = check_device();
    if (st) return st;
    dsa::RouterArgs a{logits, bias, ids, weights, T, n_experts, k, routed_scale};
    return launched(dsa::launch_router_topk(a, (hipStream_t)stream));
}

dsa_status dsa_value_up_proj(const dsa_shape* shape, const float* o, const uint16_t* wv, int32_t T, int32_t d_v,
                             uint16_t* out_v, void* stream) {
    dsa_status st = check_shape(shape);
    if (st) return st;
    if (!o || !wv || !out_v || !aligned16(o) || !aligned16(wv) || !aligned16(out_v) || T < 0 || d_v <= 0)
        return DSA_ERR_INVALID_ARG;
    if (d_v != 256 || shape->d_latent % 64 != 0) return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    if ((st = check_device())) return st;
    const int64_t H = shape->n_heads, Dl = shape->d_latent;
    dsa::GemmArgs g{o, H * Dl, Dl, wv, Dl, (int64_t)d_v * Dl, out_v, H * d_v, d_v, T, d_v, (int32_t)Dl};
    return launched(dsa::launch_value_up_proj(g, (int)H, (hipStream_t)stream));
}

dsa_status dsa_o_proj(const uint16_t* x, const uint16_t* wo, int32_t T, int32_t k_in, int32_t n_out, float* y,
                      void* stream) {
    if (!x || !wo || !y || !aligned16(x) || !aligned16(wo) || !aligned16(y) || T < 0 || k_in <= 0 || n_out <= 0)
        return DSA_ERR_INVALID_ARG;
    if (k_in % 64 != 0 || n_out % 192 != 0) return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    dsa_status st = check_device();
    if (st) return st;
    dsa::GemmArgs g{x, k_in, 0, wo, k_in, 0, y, n_out, 0, T, n_out, k_in};
    return launched(dsa::launch_o_proj(g, (hipStream_t)stream));
}

dsa_status dsa_selection_mask(const int32_t* idx, const int32_t* count, int32_t L, int32_t top_k, int32_t N,
                              int32_t q_start, int32_t mask_words, uint32_t* mask, void* stream) {
    if (!idx || !count || !mask || L < 0 || top_k <= 0 || N <= 0 || q_start < 0 ||
        (int64_t)q_start + L > INT32_MAX || (int64_t)mask_words < 2 * (((int64_t)N + 63) / 64))
        return DSA_ERR_INVALID_ARG;
    if ((int64_t)mask_words * 4 > 65536) return DSA_ERR_UNSUPPORTED;
    if (L == 0) return DSA_OK;
    dsa_status st = check_device();
    if (st) return st;
    dsa::MaskArgs a{idx, count, L, top_k, N, q_start, mask_words, mask};
    return launched(dsa::launch_selection_mask(a, (hipStream_t)stream));
}

namespace {
dsa_status dense_attn(const uint16_t* q, const uint16_t* kvb, const uint16_t* kv, int32_t kv_cols, int32_t rope_col,
                      const uint32_t* mask, int32_t mask_words, int32_t L, int32_t N, int32_t q_start, int32_t H,
                      int32_t d_nope, int32_t d_rope, int32_t d_v, float scale, float* out, const uint16_t* vt,
                      void* stream) {
    if (!q || !kvb || !kv || !mask || !out || !aligned16(q) || !aligned16(kvb) || !aligned16(kv) ||
        !aligned16(out) || ((uintptr_t)mask & 3u) || (vt && !aligned16(vt)))
        return DSA_ERR_INVALID_ARG;
    if (L < 0 || N <= 0 || H <= 0 || q_start < 0 || (int64_t)q_start + L > INT32_MAX || rope_col < 0 ||
        d_rope < 0 || (int64_t)rope_col + d_rope > kv_cols || kv_cols % 8 != 0 || rope_col % 8 != 0 ||
        (int64_t)mask_words < 2 * (((int64_t)N + 63) / 64) || !(scale > 0.f) || !std::isfinite(scale))
        return DSA_ERR_INVALID_ARG;
    int shape_id;
    if (d_nope == 192 && d_rope == 64 && d_v == 256) shape_id = 0;
    else if (d_nope == 64 && d_rope == 64 && d_v == 64) shape_id = 1;
    else return DSA_ERR_UNSUPPORTED;
    const int64_t Np = ((int64_t)N + 63) / 64 * 64;
    if ((int64_t)H * (d_nope + d_v) * 2 * 64 > INT32_MAX || (int64_t)kv_cols * 2 * 64 > INT32_MAX ||
        (int64_t)mask_words * 4 * 128 > INT32_MAX || ((int64_t)L + 127) / 128 * H > INT32_MAX ||
        (vt && d_v * Np * 2 > INT32_MAX))
        return DSA_ERR_UNSUPPORTED;
    if (L == 0) return DSA_OK;
    dsa_status st = check_device();
    if (st) return st;
    dsa::DenseArgs a{q, kvb, kv, mask, L, N, H, q_start, kv_cols, rope_col, mask_words,
                     (float)((double)scale * 1.4426950408889634), out, vt, (int32_t)Np};
    return launched(dsa::launch_dense_attn(shape_id, a, (hipStream_t)stream));
}
}  // namespace

dsa_status dsa_dense_masked_attn(const uint16_t* q, const uint16_t* kvb, const uint16_t* kv, int32_t kv_cols,
                                 int32_t rope_col, const uint32_t* mask, int32_t mask_words, int32_t L,
                                 int32_t N, int32_t q_start, int32_t H, int32_t d_nope, int32_t d_rope,
                                 int32_t d_v, float scale, float* out, void* stream) {
    return dense_attn(q, kvb, kv, kv_cols, rope_col, mask, mask_words, L, N, q_start, H, d_nope, d_rope, d_v,
                      scale, out, nullptr, stream);
}

dsa_status dsa_dense_masked_attn_f16(const uint16_t* q, const uint16_t* kvb, const uint16_t* vt, const uint16_t* kv,
                                     int32_t kv_cols, int32_t rope_col, const uint32_t* mask, int32_t mask_words,
                                     int32_t L, int32_t N, int32_t q_start, int32_t H, int32_t d_nope,
                                     int32_t d_rope, int32_t d_v, float scale, float* out, void* stream) {
    if (!vt) return DSA_ERR_INVALID_ARG;
    return dense_attn(q, kvb, kv, kv_cols, rope_col, mask, mask_words, L, N, q_start, H, d_nope, d_rope, d_v,
                      scale, out, vt, stream);
}

dsa_status dsa_values_to_f16(const uint16_t* kvb, int32_t N, int32_t H, int32_t d_nope, int32_t d_v, uint16_t* vt,
                             void* stream) {
    if (!kvb || !vt || !aligned16(kvb) || !aligned16(vt) || N < 0 || H <= 0 || d_nope < 0 || d_nope % 8 != 0)
        return DSA_ERR_INVALID_ARG;
    if (d_v != 256 && d_v != 64) return DSA_ERR_UNSUPPORTED;
    const int64_t Np = ((int64_t)N + 63) / 64 * 64;
    if (Np > INT32_MAX || H > 65535) return DSA_ERR_UNSUPPORTED;   // grid (Np / 64, H)
    if (N == 0) return DSA_OK;
    dsa_status st = check_device();
    if (st) return st;
    return launched(dsa::launch_values_to_vt(kvb, N, H, d_nope, d_v, (int)Np, vt, (hipStream_t)stream));
}

dsa_status dsa_kv_b_proj(const uint16_t* kv, int32_t kv_cols, const uint16_t* wkvb, int32_t N, int32_t H,
                         int32_t d_latent, int32_t d_nope, int32_t d_v, uint16_t* kvb, uint16_t* vt,
                         void* stream) {
    if (!kv || !wkvb || !kvb || !aligned16(kv) || !aligned16(wkvb) || !aligned16(kvb) || (vt && !aligned16(vt)) ||
        N < 0 || H <= 0 || d_latent <= 0 || d_latent > kv_cols || kv_cols % 8 != 0 || d_nope < 0 || d_v <= 0)
        return DSA_ERR_INVALID_ARG;
    const int64_t n_out = (int64_t)H * (d_nope + d_v);
    if (d_latent % 64 != 0 || n_out % 256 != 0 || n_out > INT32_MAX || (int64_t)N * kv_cols * 2 >= (1ll << 32) ||
        n_out * d_latent * 2 >= (1ll << 32))
        return DSA_ERR_UNSUPPORTED;
    if (N == 0) return DSA_OK;
    dsa_status st = check_device();
    if (st) return st;
    const int64_t Np = ((int64_t)N + 63) / 64 * 64;
    if (vt && (int64_t)H * d_v * Np >= ((int64_t)1 << 40)) return DSA_ERR_UNSUPPORTED;
    dsa::GemmArgs g{kv, kv_cols, 0, wkvb, d_latent, 0, kvb, n_out, 0, N, (int32_t)n_out, d_latent};
    if (vt) {
        g.vt = vt;
        g.vt_from = d_nope;
        g.vt_period = d_nope + d_v;
        g.vt_np = (int32_t)Np;
    }
    return launched(dsa::launch_kv_b_proj(g, (hipStream_t)stream));
}

dsa_status dsa_absorb_weight(const uint16_t* wkvb, int32_t H, int32_t d_nope, int32_t d_v, int32_t d_latent,
                             uint16_t* wk_t, void* stream) {
    if (!wkvb || !wk_t || H <= 0 || d_nope <= 0 || d_v < 0 || d_latent <= 0) return DSA_ERR_INVALID_ARG;
    if ((int64_t)H * (d_nope + d_v) * d_latent >= ((int64_t)1 << 40)) return DSA_ERR_UNSUPPORTED;
    dsa_status st = check_device();
    if (st) return st;
    return launched(dsa::launch_absorb_weight(wkvb, H, d_nope, d_v, d_latent, wk_t, (hipStream_t)stream));
}

dsa_status dsa_q_absorb(const uint16_t* q, const uint16_t* wk_t, int32_t T, int32_t H, int32_t d_nope,
                        int32_t d_rope, int32_t d_latent, uint16_t* q_abs, void* stream) {
    if (!q || !wk_t || !q_abs || !aligned16(q) || !aligned16(wk_t) || !aligned16(q_abs) || T < 0 || H <= 0 ||
        d_nope <= 0 || d_rope < 0 || d_latent <= 0)
        return DSA_ERR_INVALID_ARG;
    const int64_t qc = (int64_t)d_nope + d_rope, oc = (int64_t)d_latent + d_rope;
    if (d_nope % 64 != 0 || d_latent % 256 != 0 || d_rope % 8 != 0 || (int64_t)T * H * qc * 2 >= (1ll << 32) ||
        (int64_t)d_latent * d_nope * 2 >= (1ll << 32))
        return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    dsa_status st = check_device();
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    dsa::GemmArgs g{q, H * qc, qc, wk_t, d_nope, (int64_t)d_latent * d_nope, q_abs, H * oc, oc,
                    T, d_latent, d_nope};
    if ((st = launched(dsa::launch_q_absorb(g, H, s)))) return st;
    return launched(dsa::launch_copy_cols(q, qc, d_nope, q_abs, oc, d_latent, (int64_t)T * H, d_rope, s));
}

dsa_status dsa_sparse_mla_attn_f16(const dsa_shape* shape, const uint16_t* q, const uint16_t* kv16,
                                   const int32_t* idx, const int32_t* count, int32_t L, int32_t N,
                                   float* out, float* lse, void* stream) {
    dsa_status st = check_shape(shape);
    if (st) return st;
    if (!q || !kv16 || !idx || !count || !out || !aligned16(q) || !aligned16(kv16) || !aligned16(out) ||
        (lse && !aligned16(lse)))
        return DSA_ERR_INVALID_ARG;
    if (L <= 0 || N <= 0) return DSA_ERR_INVALID_ARG;
    if (!attn_keys_ok(shape, N)) return DSA_ERR_UNSUPPORTED;
    if ((st = check_device())) return st;
    dsa::AttnArgs a{q, kv16, idx, count, L, N, shape->top_k, scale_log2(shape), out, lse};
    return launched(dsa::launch_attention(shape_id(shape), a, true, (hipStream_t)stream));
}

size_t dsa_prefill_workspace_bytes(const dsa_shape* shape, int32_t L, int32_t N, int64_t q_start) {
    if (check_shape(shape) != DSA_OK || L <= 0 || q_start < 0 || (int64_t)N != q_start + L) return 0;
    return prefill_layout(shape, L, N, q_start).total;
}

dsa_status dsa_prefill_chunk(const dsa_shape* shape, const uint16_t* q, const uint16_t* qI,
                             const float* w, const uint16_t* kv, const uint16_t* kI, int32_t L,
                             int32_t N, int64_t q_start, float* out, int32_t* idx_out,
                             int32_t* count_out, void* ws, size_t ws_bytes, void* stream) {
    dsa_status st = check_shape(shape);
    if (st) return st;
    if (!q || !qI || !w || !kv || !kI || !out)
        return DSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(qI) || !aligned16(w) || !aligned16(kv) || !aligned16(kI) ||
        !aligned16(out) || (idx_out && !aligned16(idx_out)) || (count_out && !aligned16(count_out)))
        return DSA_ERR_INVALID_ARG;
    if (L <= 0 || q_start < 0 || (int64_t)N != q_start + L) return DSA_ERR_INVALID_ARG;
    if (N > dsa::kMaxSelectKeys) return DSA_ERR_UNSUPPORTED;
    const PrefillLayout lay = prefill_layout(shape, L, N, q_start);
    if (!ws || !aligned16(ws) || ws_bytes < lay.total) return DSA_ERR_WORKSPACE;
    if ((st = check_device())) return st;
    hipStream_t s = (hipStream_t)stream;
    const int sid = shape_id(shape);
    char* base = static_cast<char*>(ws);
    float* S = reinterpret_cast<float*>(base + lay.s_off);
    int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + lay.idx_off);
    int32_t* cnt = count_out ? count_out : reinterpret_cast<int32_t*>(base + lay.cnt_off);
    const int64_t dq = (int64_t)shape->n_idx_heads * shape->d_idx;

    // 1. indexer scores for the queries with more causal keys than top_k
    dsa::IndexerArgs ia{qI + lay.row0 * dq, kI, w + (int64_t)lay.row0 * shape->n_idx_heads, S, lay.ldS,
                        L - lay.row0, N, q_start + lay.row0, 0};
    if ((st = launched(dsa::launch_indexer_prefill(sid, ia, s)))) return st;
    // 2. selection (every earlier key below the boundary)
    dsa::TopkArgs ta{S, lay.ldS, lay.row0, L, q_start, shape->top_k, idx, cnt};
    if ((st = launched(dsa::launch_topk_prefill(ta, N, s)))) return st;
    // 3. attention over the gathered rows, on an fp16-latent copy of the
    //    cache (converted once per chunk, read by every query)
    uint16_t* kv16 = reinterpret_cast<uint16_t*>(base + lay.kv16_off);
    if ((st = launched(dsa::launch_latent_to_f16(sid, kv, kv16, N, s)))) return st;
    dsa::AttnArgs aa{q, kv16, idx, cnt, L, N, shape->top_k, scale_log2(shape), out, nullptr};
    return launched(dsa::launch_attention(sid, aa, true, s));
}

size_t dsa_decode_workspace_bytes(const dsa_shape* shape, int32_t B, const int64_t* ctx) {
    if (check_shape(shape) != DSA_OK) return 0;
    size_t need = 0;
    return decode_need(shape, B, ctx, need) == DSA_OK ? need : 0;
}

dsa_status dsa_decode_step(const dsa_shape* shape, int32_t B, const int64_t* ctx,
                           const uint16_t* q, const uint16_t* qI, const float* w,
                           const uint16_t* kv, const uint16_t* kI, float* out, int32_t* idx_out,
                           int32_t* count_out, void* ws, size_t ws_bytes, void* stream) {
    size_t need = 0;
    dsa_status st = decode_check(shape, B, ctx, q, qI, w, kv, kI, out, idx_out, count_out, need);
    if (st) return st;
    if (!ws || !aligned16(ws) || ws_bytes < need) return DSA_ERR_WORKSPACE;
    if ((st = check_device())) return st;
    return decode_groups(shape, B, ctx, q, qI, w, kv, kI, out, idx_out, count_out, static_cast<char*>(ws),
                         (hipStream_t)stream);
}

dsa_status dsa_decode_step_noalloc(const dsa_shape* shape, int32_t B, const int64_t* ctx,
                                   const uint16_t* q, const uint16_t* qI, const float* w,
                                   const uint16_t* kv, const uint16_t* kI, float* out, int32_t* idx_out,
                                   int32_t* count_out, void* stream) {
    size_t need = 0;
    dsa_status st = decode_check(shape, B, ctx, q, qI, w, kv, kI, out, idx_out, count_out, need);
    if (st) return st;
    if (need > DSA_DECODE_STATIC_SCRATCH_BYTES) return DSA_ERR_WORKSPACE;
    if ((st = check_device())) return st;
    void* scratch_dev = nullptr;
    if ((st = static_scratch(&scratch_dev))) return st;
    return decode_groups(shape, B, ctx, q, qI, w, kv, kI, out, idx_out, count_out, static_cast<char*>(scratch_dev),
                         (hipStream_t)stream);
}

}  // extern "C"
