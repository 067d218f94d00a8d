// indexer.hip - DSA indexer scores on gfx950 MFMA.
//
// exo PR #2539 (glm_moe_dsa attention speed-ups), Prefill section, float32
// indexer item: a key's score for a query is the sum over the indexer heads
// of the head weight times relu(q.k), accumulated in float32 in one pass with
// the causal mask applied.  One Di-wide indexer key per token is shared by
// all heads.
//
// Design: the product for one query is a [heads x Di] x [Di x keys] GEMM, so
// the 32 indexer heads are the 32 rows of a v_mfma_f32_32x32x16_bf16 tile and
// 32 keys its columns.  In the 32x32 accumulator layout a lane holds 16 of
// the 32 heads of one key, so the weighted relu sum over heads is 16 FMAs in
// the lane plus one exchange with lane l^32 (v_permlane32_swap), which also
// packs two results per lane.  bf16 products of integers are exact and the
// fp32 sum is exact while it stays below 2^24.
//
// Prefill: a block holds 16 queries (2 per wave, their Q fragments and
// weights stay in VGPRs) and streams a 1024-key tile through LDS in 64-key
// double-buffered sub-tiles, so each key row is read from L2 once per 16
// queries.  Tiles past the block's last causal key are not computed.
// Decode: one query per sequence, so no reuse across queries: each wave reads
// its keys straight from memory into MFMA operands (the step is HBM bound).
#include "dsa_kernels.h"

#include <math.h>

namespace dsa {
namespace {

template <int HI, int DI>
struct IdxShape {
    static_assert(HI <= 32 && HI % 4 == 0, "indexer heads must fit one 32-row MFMA tile");
    static_assert(DI % 16 == 0, "indexer width must be a multiple of the MFMA K step");
    static constexpr int KS = DI / 16;        // 32x32x16 K steps
    static constexpr int ROWB = DI * 2 + 16;  // LDS bytes per key row, padded against bank conflicts
    static constexpr int CPR = DI / 8;        // 16-byte pieces per key row
};

constexpr int kIdxWaves = 8;
constexpr int kIdxThreads = kIdxWaves * 64;
constexpr int kIdxQPB = kIdxWaves * 2;   // queries per block
constexpr int kIdxSub = 64;              // keys per LDS sub-tile
constexpr int kIdxTile = 1024;           // keys per block

constexpr int kIdxdWaves = 4;
constexpr int kIdxdKeysPerWave = 128;
constexpr int kIdxdKeysPerBlock = kIdxdWaves * kIdxdKeysPerWave;

// Head held by accumulator register r of lane-half `half` in the 32x32 layout.
__device__ inline int acc_head(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

template <int HI, int DI>
__device__ inline void load_query(const uint16_t* qI, const float* w, int64_t q, bool valid,
                                  int col, int half, u32x4 (&qf)[IdxShape<HI, DI>::KS],
                                  float (&wr)[16]) {
    using C = IdxShape<HI, DI>;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
        qf[ks] = (valid && col < HI) ? ldg16(qI + (q * HI + col) * DI + ks * 16 + half * 8) : zero;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int h = acc_head(r, half);
        wr[r] = (valid && h < HI) ? w[q * HI + h] : 0.f;
    }
}

// sum over this lane's 16 heads of w * relu(score)
__device__ inline float weighted_relu(const f32x16& acc, const float (&wr)[16]) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s = fmaf(wr[r], fmaxf(acc[r], 0.f), s);
    return s;
}

// lanes 0-31 get x summed over both halves, lanes 32-63 get y summed likewise
__device__ inline float combine_halves(float x, float y) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int HI, int DI>
__global__ __launch_bounds__(kIdxThreads) __attribute__((amdgpu_waves_per_eu(2)))
void indexer_prefill_kernel(IndexerArgs a) {
    using C = IdxShape<HI, DI>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[2][kIdxSub * C::ROWB];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, col = lane & 31;
    const int q_base = blockIdx.y * kIdxQPB;
    if (q_base >= a.rows) return;
    const int q_last = min(q_base + kIdxQPB, a.rows) - 1;
    const int64_t p_last = a.pos0 + q_last;
    const int key_beg = blockIdx.x * kIdxTile;
    const int key_tile_end = min(key_beg + kIdxTile, a.N);
    const int kend = (int)min<int64_t>((int64_t)key_tile_end, p_last + 1);

    if (a.write_masked) {   // keys every query of the block masks
        const int m0 = max(kend, key_beg);
        const int width = key_tile_end - m0;
        if (width > 0) {
            const int n = (q_last - q_base + 1) * width;
            for (int e = tid; e < n; e += kIdxThreads)
                a.S[(int64_t)(q_base + e / width) * a.ldS + m0 + e % width] = -INFINITY;
        }
    }
    if (kend <= key_beg) return;

    const int qa = q_base + 2 * wave, qb = qa + 1;
    const bool va = qa < a.rows, vb = qb < a.rows;
    const int64_t pa = a.pos0 + qa, pb = a.pos0 + qb;
    const int64_t pmax = vb ? pb : pa;

    u32x4 qfa[C::KS], qfb[C::KS];
    float wa[16], wb[16];
    load_query<HI, DI>(a.qI, a.w, qa, va, col, half, qfa, wa);
    load_query<HI, DI>(a.qI, a.w, qb, vb, col, half, qfb, wb);

    constexpr int CH = kIdxSub * C::CPR;
    constexpr int CPT = (CH + kIdxThreads - 1) / kIdxThreads;
    u32x4 stage[CPT];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto gload = [&](int s) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int ci = tid + c * kIdxThreads;
            const int j = key_beg + s * kIdxSub + ci / C::CPR;
            stage[c] = (ci < CH && j < a.N) ? ldg16(a.kI + (int64_t)j * DI + (ci % C::CPR) * 8) : zero;
        }
    };
    auto swrite = [&](int buf) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int ci = tid + c * kIdxThreads;
            if (ci < CH)
                *reinterpret_cast<u32x4*>(&lds[buf][(ci / C::CPR) * C::ROWB + (ci % C::CPR) * 16]) = stage[c];
        }
    };

    const int nsub = (kend - key_beg + kIdxSub - 1) / kIdxSub;
    gload(0);
    swrite(0);
    __syncthreads();
    for (int s = 0; s < nsub; ++s) {
        if (s + 1 < nsub) gload(s + 1);
        const unsigned char* buf = lds[s & 1];
#pragma unroll
        for (int c = 0; c < kIdxSub / 32; ++c) {
            const int jc = key_beg + s * kIdxSub + 32 * c;
            if (!va || jc >= kend) continue;
            const int key = jc + col;
            const int q = half ? qb : qa;
            const bool vq = half ? vb : va;
            const int64_t p = half ? pb : pa;
            if (jc > pmax) {   // every key of the chunk is past both queries
                if (a.write_masked && vq && key < kend) a.S[(int64_t)q * a.ldS + key] = -INFINITY;
                continue;
            }
            u32x4 bf[C::KS];
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                bf[ks] = *reinterpret_cast<const u32x4*>(buf + (32 * c + col) * C::ROWB + ks * 32 + half * 16);
            f32x16 acca = {}, accb = {};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                acca = mfma32_bf16(qfa[ks], bf[ks], acca);
                accb = mfma32_bf16(qfb[ks], bf[ks], accb);
            }
            const float tot = combine_halves(weighted_relu(acca, wa), weighted_relu(accb, wb));
            if (vq && key < kend) {
                if (key <= p) a.S[(int64_t)q * a.ldS + key] = tot;
                else if (a.write_masked) a.S[(int64_t)q * a.ldS + key] = -INFINITY;
            }
        }
        if (s + 1 < nsub) swrite((s + 1) & 1);
        __syncthreads();
    }
}

template <int HI, int DI>
__global__ __launch_bounds__(kIdxdWaves * 64)
void indexer_decode_kernel(const uint16_t* __restrict__ qI, const uint16_t* __restrict__ kI,
                           const float* __restrict__ w, float* __restrict__ S, SeqMeta m) {
    using C = IdxShape<HI, DI>;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, col = lane & 31;
    const int b = seq_of_block(m, blockIdx.x);
    const int ctx = m.ctx[b];
    const int kb = (blockIdx.x - m.blk0[b]) * kIdxdKeysPerBlock + wave * kIdxdKeysPerWave;
    if (kb >= ctx) return;

    u32x4 qf[C::KS];
    float wr[16];
    load_query<HI, DI>(qI, w, b, true, col, half, qf, wr);
    const uint16_t* kbase = kI + m.key_off[b] * DI;
    float* srow = S + m.s_off[b];
    const u32x4 zero = {0u, 0u, 0u, 0u};

#pragma unroll
    for (int c = 0; c < kIdxdKeysPerWave / 32; c += 2) {
        const int j0 = kb + 32 * c + col, j1 = j0 + 32;
        u32x4 b0[C::KS], b1[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            b0[ks] = j0 < ctx ? ldg16(kbase + (int64_t)j0 * DI + ks * 16 + half * 8) : zero;
            b1[ks] = j1 < ctx ? ldg16(kbase + (int64_t)j1 * DI + ks * 16 + half * 8) : zero;
        }
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            acc0 = mfma32_bf16(qf[ks], b0[ks], acc0);
            acc1 = mfma32_bf16(qf[ks], b1[ks], acc1);
        }
        const float tot = combine_halves(weighted_relu(acc0, wr), weighted_relu(acc1, wr));
        const int key = kb + 32 * (c + half) + col;
        if (key < ctx) srow[key] = tot;   // the query sits at ctx-1: every cached key is visible
    }
}

}  // namespace

int indexer_decode_keys_per_block() { return kIdxdKeysPerBlock; }

hipError_t launch_indexer_prefill(int shape_id, const IndexerArgs& a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    dim3 grid((a.N + kIdxTile - 1) / kIdxTile, (a.rows + kIdxQPB - 1) / kIdxQPB);
    if (shape_id == 0)
        hipLaunchKernelGGL((indexer_prefill_kernel<32, 128>), grid, dim3(kIdxThreads), 0, s, a);
    else
        hipLaunchKernelGGL((indexer_prefill_kernel<4, 32>), grid, dim3(kIdxThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_indexer_decode(int shape_id, const uint16_t* qI, const uint16_t* kI,
                                 const float* w, float* S, const SeqMeta& m, int blocks,
                                 hipStream_t s) {
    if (blocks <= 0) return hipSuccess;
    if (shape_id == 0)
        hipLaunchKernelGGL((indexer_decode_kernel<32, 128>), dim3(blocks), dim3(kIdxdWaves * 64), 0, s,
                           qI, kI, w, S, m);
    else
        hipLaunchKernelGGL((indexer_decode_kernel<4, 32>), dim3(blocks), dim3(kIdxdWaves * 64), 0, s,
                           qI, kI, w, S, m);
    return hipGetLastError();
}

}  // namespace dsa
