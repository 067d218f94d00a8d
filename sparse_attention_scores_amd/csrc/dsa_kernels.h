// dsa_kernels.h - internal to the HIP library: device types, helpers and the
// launcher entry points the C ABI (dsa_api.hip) calls.  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxBatch = 128;      // decode sequences per step
constexpr int kMaxTopK = 2048;
constexpr int kMaxSelectKeys = 1 << 18;   // keys one selection may read (262144)

// Per-sequence geometry of a decode step, passed by value in kernel
// arguments so that no host-to-device copy is needed.
struct SeqMeta {
    int32_t B;
    int32_t pad_;
    int64_t key_off[kMaxBatch + 1];   // first cache row of sequence b
    int64_t s_off[kMaxBatch + 1];     // first score of sequence b (64-aligned)
    int32_t ctx[kMaxBatch];           // keys of sequence b; query at ctx-1
    int32_t blk0[kMaxBatch + 1];      // first block of sequence b (per kernel)
};

// Which sequence owns block `blk`: the last b with blk0[b] <= blk (blk0 is
// ascending and blk0[0] = 0), by bisection, so a block waits on log2(B)
// dependent scalar loads rather than up to B.
__device__ inline int seq_of_block(const SeqMeta& m, int blk) {
    int lo = 0, n = m.B;   // the answer lies in [lo, lo + n)
    while (n > 1) {
        const int h = n >> 1;
        const bool up = blk >= m.blk0[lo + h];
        lo = up ? lo + h : lo;
        n = up ? n - h : h;
    }
    return lo;
}

__device__ inline f32x4 mfma16_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ inline f32x4 mfma16_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ inline f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ inline f32x16 mfma32_f16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ inline u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two fp16 in one dword (a in the low half), rounded to
// nearest even (v_cvt_pk_f16_f32).  Unbiased: a probability rounded this way
// keeps the value product's numerator and the fp32 denominator consistent
// on average, where truncation would scale every output down by about 2^-11.
__device__ inline uint32_t pack_f16_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// ---- wave primitives on DPP (every lane of the wave active) ----
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within each 16-lane row

// A permutation inside each 16-lane row: every lane has a source.
template <int CTRL>
__device__ inline int dpp_perm(int x) {
    return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xf, 0xf, false);
}

// Sum over aligned groups of P lanes (P a power of two up to 16, uniform):
// after the two quad exchanges every lane holds its quad's sum, and each
// mirror adds the group it is paired with.
__device__ inline int group_sum(int x, int P) {
    if (P >= 2) x += dpp_perm<kDppXor1>(x);
    if (P >= 4) x += dpp_perm<kDppXor2>(x);
    if (P >= 8) x += dpp_perm<kDppHalfMirror>(x);
    if (P >= 16) x += dpp_perm<kDppMirror>(x);
    return x;
}

#define DSA_LDS __attribute__((address_space(3)))

__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const DSA_LDS void*)p;
}

// 16 bytes per lane from base + voff (a uniform 64-bit base, a per-lane
// 32-bit offset) to LDS at m0 + 16 * lane, without passing through VGPRs.
// Completion is counted by vmcnt only: the compiler does not see these
// loads, so the kernel waits for them itself (wait_vmcnt) before a barrier.
// M0 is written here and in load4_to_lds, nowhere else in these kernels.
__device__ inline void gather16_to_lds(const void* base, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(base) : "memory");
}

// 4 bytes per lane from base + voff to LDS at m0 + 4 * lane; otherwise as
// gather16_to_lds (counted by vmcnt only, M0 written here).
__device__ inline void load4_to_lds(const void* base, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(base) : "memory");
}

template <int N>
__device__ inline void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// ---- launchers (each returns hipGetLastError() of its launches) ----------

struct IndexerArgs {
    const uint16_t* qI;   // [rows, Hi, Di]  (row r = query row0 + r)
    const uint16_t* kI;   // [N, Di]
    const float* w;       // [rows, Hi]
    float* S;             // [rows, ldS]
    int64_t ldS;
    int32_t rows;         // queries scored
    int32_t N;            // keys
    int64_t pos0;         // position of the first scored query
    int32_t write_masked; // also write -inf for keys past each query
    int32_t key_tile;     // keys per block (set by the launcher)
};
// Shape ids: 0 = GLM (Hi 32, Di 128), 1 = tiny (Hi 4, Di 32)
hipError_t launch_indexer_prefill(int shape_id, const IndexerArgs& a, hipStream_t s);
hipError_t launch_indexer_decode(int shape_id, const uint16_t* qI, const uint16_t* kI,
                                 const float* w, float* S, const SeqMeta& m, int blocks,
                                 hipStream_t s);
int indexer_decode_keys_per_block();

struct TopkArgs {
    const float* S;       // prefill: row r at S + (r - s_row0) * ldS
    int64_t ldS;
    int32_t s_row0;       // first row that has scores (earlier rows are dense)
    int32_t rows;
    int64_t pos0;         // position of row 0
    int32_t top_k;
    int32_t* idx;         // [rows, top_k]
    int32_t* count;       // [rows] or null
};
hipError_t launch_topk_prefill(const TopkArgs& a, int n_max, hipStream_t s);
// Decode top-k: m.blk0 numbers the segment blocks of each sequence
// (topk_decode_segments(ctx, top_k) each: none for a sequence of at most
// top_k keys); `work` holds topk_decode_work_bytes(B, blocks, top_k) bytes.
// The two launches leave, per sequence of more than top_k keys, either its
// selection in idx/count (the fallback: info.degenerate or info.fallback
// set) or the lists the decode attention merges: `above` sure keys and
// `inbin` candidates, of which the top_k - above best (score, then lower
// key) are kept.
constexpr int kDecCap = 1024;                 // boundary-bin keys a sequence may leave as candidates
struct DecCand {        // a boundary-bin key of a sequence and its score (NaN as -inf)
    int32_t key;
    float score;
};
struct DecSeqInfo {     // per sequence
    float scale, off;   // the shared map: bin(v) = clamp(trunc(v * scale + off), 0, kDecBins - 1)
    int degenerate;     // the sample gave no usable range
    int fallback;       // the boundary bin holds more than kDecCap keys
    int above, inbin;   // keys in bins above the boundary bin; keys in it
    int pad_[2];
};
struct DecWork {
    int* hist;          // [segment block][kDecBins]
    DecSeqInfo* info;   // [B]
    int32_t* sure;      // [B][top_k]: keys above the boundary bin, ascending
    DecCand* cand;      // [B][kDecCap]: keys in it, ascending
};
int topk_decode_segments(int ctx, int top_k);
size_t topk_decode_work_bytes(int B, int blocks, int top_k);
DecWork topk_decode_work(void* work, int B, int blocks, int top_k);
hipError_t launch_topk_decode(const float* S, const SeqMeta& m, int top_k, int32_t* idx,
                              int32_t* count, void* work, hipStream_t s);

struct AttnArgs {
    const uint16_t* q;     // [rows, H, Dqk]
    const uint16_t* kv;    // [N, Dqk] (decode: packed caches)
    const int32_t* idx;    // [rows, top_k]
    const int32_t* count;  // [rows]
    int32_t rows;
    int32_t N;
    int32_t top_k;
    float scale_log2;      // softmax_scale * log2(e)
    float* out;            // [rows, H, Dl]
    float* lse;            // [rows, H] or null
};
// Split (decode) variant: block -> (sequence, chunk of `chunk` selected keys);
// writes unnormalised partial outputs, then a combine kernel finishes.  The
// blocks also finish the selection: each takes its chunk of the ascending
// selection (merging the top-k lists in `dec`, or every key of a sequence of
// at most top_k keys, or the fallback's idx) and writes it to idx; the first
// chunk of a sequence writes its count and padding.
struct AttnSplitArgs {
    const uint16_t* q;
    const uint16_t* kv;
    int32_t* idx;          // [B, top_k]
    int32_t* count;        // [B]
    DecWork dec;
    int32_t top_k;
    int32_t chunk;
    float scale_log2;
    float* part_o;         // [items, H, Dl]
    float* part_ml;        // [items, H, 2] (running max in log2 units, sum)
    float* out;            // [B, H, Dl]
};
// kv_f16: the cache's latent columns are fp16 (launch_latent_to_f16 output)
hipError_t launch_attention(int shape_id, const AttnArgs& a, bool kv_f16, hipStream_t s);
hipError_t launch_latent_to_f16(int shape_id, const uint16_t* kv, uint16_t* kv16, int64_t rows, hipStream_t s);
hipError_t launch_attention_split(int shape_id, const AttnSplitArgs& a, const SeqMeta& m,
                                  int items, hipStream_t s);

struct CacheWriteArgs {
    const uint16_t* kv_a;    // [T, Dl+Dr] new rows [kv_cmpr | k_pe]
    const float* norm_w;     // [Dl]
    const int32_t* pos;      // [T]
    const uint16_t* kI_new;  // [T, Di] or null
    uint16_t* kv;            // [N, Dl+Dr] latent cache
    uint16_t* kI;            // [N, Di] indexer cache or null
    uint16_t* q;             // [T, H, Dl+Dr] or null (rope columns rotated in place)
    uint16_t* qI;            // [T, Hi, Di] or null (leading d_idx_rope columns rotated)
    int32_t T, N, d_idx_rope;
    float eps, theta;
};
hipError_t launch_cache_write(int shape_id, const CacheWriteArgs& a, hipStream_t s);

struct RouterArgs {
    const float* logits;     // [T, E]
    const float* bias;       // [E]
    int32_t* ids;            // [T, k]
    float* weights;          // [T, k]
    int32_t T, E, k;
    float scale;
};
// E in {64, 128, 256, 512, 1024}, 1 <= k <= min(32, E)
hipError_t launch_router_topk(const RouterArgs& a, hipStream_t s);

struct GemmArgs {            // C[m, n] = sum_k A[m, k] B[n, k], per batch z
    const void* A;           // element (z, m, k) at z*a_batch + m*lda + k (float32 or bf16)
    int64_t lda, a_batch;
    const uint16_t* B;       // bf16, element (z, n, k) at z*b_batch + n*ldb + k
    int64_t ldb, b_batch;
    void* C;                 // element (z, m, n) at z*c_batch + m*ldc + n (bf16 or float32)
    int64_t ldc, c_batch;
    int32_t M, N, K;
    // bf16 output only, the kv_b value form: column n with
    // n % vt_period >= vt_from goes to vt[n / vt_period][n % vt_period -
    // vt_from][.] in fp16 (keys in the dense tile order, stride vt_np, rows
    // from M up to vt_np written as zeros) instead of to C
    uint16_t* vt = nullptr;
    int32_t vt_from = 0, vt_period = 0, vt_np = 0;
};
// value up-projection: A float32, C bf16, N == 256, K % 64 == 0
hipError_t launch_value_up_proj(const GemmArgs& g, int batch, hipStream_t s);
// output projection: A bf16, C float32, N % 192 == 0, K % 64 == 0
hipError_t launch_o_proj(const GemmArgs& g, hipStream_t s);
// kv_b up-projection: A bf16 (latent rows), C bf16 / fp16 columns, N % 256 == 0, K % 64 == 0
hipError_t launch_kv_b_proj(const GemmArgs& g, hipStream_t s);
// query absorption: A = q no-rope columns (bf16), B = transposed key block,
// C bf16, batch = heads (grid z); N % 256 == 0, K % 64 == 0
hipError_t launch_q_absorb(const GemmArgs& g, int batch, hipStream_t s);
// dst[r, dst_col0 + c] = src[r, src_col0 + c], c < ncols (bf16, 16-byte chunks)
hipError_t launch_copy_cols(const uint16_t* src, int64_t src_ld, int src_col0, uint16_t* dst, int64_t dst_ld,
                            int dst_col0, int64_t rows, int ncols, hipStream_t s);
// wkT[h, d, c] = w[h*(Dn+Dv) + c, d]
hipError_t launch_absorb_weight(const uint16_t* w, int H, int Dn, int Dv, int Dl, uint16_t* wkT, hipStream_t s);

// Selection mask: row i of mask [L, W] has bit j set iff key j is among
// idx[i, :count[i]], 0 <= j < N and j <= q_start + i.
struct MaskArgs {
    const int32_t* idx;    // [L, top_k]
    const int32_t* count;  // [L]
    int32_t L, top_k, N, q_start, W;
    uint32_t* mask;        // [L, W]
};
hipError_t launch_selection_mask(const MaskArgs& a, hipStream_t s);

// Dense masked attention, non-absorbed form: per head, one (Dn + Dr)-wide
// score product against [no-rope key | shared rope key], keys limited to
// the mask bits, values the head's Dv columns of kvb.
struct DenseArgs {
    const uint16_t* q;      // [L, H, Dn + Dr]
    const uint16_t* kvb;    // [N, H, Dn + Dv]
    const uint16_t* kv;     // [N, kv_cols]; rope key at columns rope_col ..
    const uint32_t* mask;   // [L, W]
    int32_t L, N, H, q_start, kv_cols, rope_col, W;
    float scale_log2;       // softmax_scale * log2(e)
    float* out;             // [L, H, Dv]
    const uint16_t* vt;     // fp16 values [H][Dv][Np] in the tile key order, or null: bf16 values in kvb
    int32_t Np;             // vt's key stride: N rounded up to 64
};
hipError_t launch_dense_attn(int shape_id, const DenseArgs& a, hipStream_t s);
// The value columns of kvb [N, H, Dn + Dv] -> vt [H][Dv][Np] fp16 (tile key order, zero past N).
hipError_t launch_values_to_vt(const uint16_t* kvb, int N, int H, int dn, int dv, int Np, uint16_t* vt,
                               hipStream_t s);

}  // namespace dsa
