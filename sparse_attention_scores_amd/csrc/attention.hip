// attention.hip - absorbed-MLA attention over gathered latent rows on gfx950.
//
// Pipeline trace ("GLM-5.2-Vision: llama.cpp vs vLLM"), section 6: the query
// is [q_nope_absorbed | q_pe] (Dl + Dr wide), every head scores the shared
// latent key row [kv_cmpr | k_pe], the value is kv_cmpr (the first Dl
// columns), softmax with kq_scale.  exo PR #2539, Prefill section: each query
// gathers its selected latent rows with 16-byte vector copies and runs a
// float32 softmax over them; Decode section: the heads are the rows of one
// product with the shared latent keys.
//
// Design (one block = one query, or one chunk of a query's selection):
//  - 32 selected rows per tile are gathered with 16-byte loads (a row is 1152
//    bytes at GLM shape) and staged in LDS twice: row-major bf16 for the
//    score product and transposed fp16 for the value product.  The
//    transpose happens in registers (8 keys x 8 features per thread), so
//    both products read their MFMA operands with 16-byte LDS loads.
//  - wave w owns heads 16w..16w+15.  Scores are S^T = K Q^T on
//    v_mfma_f32_16x16x32_bf16 with the queries' fragments held in VGPRs; the
//    output O^T = V^T P^T runs on v_mfma_f32_16x16x32_f16 with the O
//    accumulators in VGPRs.  The key order inside a 32-key tile is permuted in
//    the transposed copy so that the score accumulators of a lane are exactly
//    its probability operand: no shuffles between the two products.
//  - online softmax in fp32 in base 2; the output rescale is skipped when no
//    head's running maximum moved.
//  - probabilities enter the value product as fp16 (11-bit significand): a
//    bf16 probability operand would cost about 1.5e-3 relative error on its
//    own; the latent values are exact in fp16 for |v| <= 65504.
#include "dsa_kernels.h"

#include <math.h>

namespace dsa {
namespace {

constexpr int kTK = 32;   // keys per tile

template <int NH, int DL, int DR>
struct AttnShape {
    static_assert(DL % 16 == 0 && DR % 8 == 0, "latent widths must be multiples of 16 / 8");
    static constexpr int NW = (NH + 15) / 16;            // waves: 16 heads each
    static constexpr int NT = NW * 64;
    static constexpr int DQK = DL + DR;
    static constexpr int DQKP = (DQK + 31) / 32 * 32;    // score K dim padded to the MFMA step
    static constexpr int KS = DQKP / 32;                 // score K steps
    static constexpr int FB = DL / 16;                   // value feature blocks
    static constexpr int KROW = DQKP * 2 + 16;           // LDS bytes per key row (padded)
    static constexpr int VROW = kTK * 2 + 16;            // LDS bytes per transposed value row
    static constexpr int LDS_K = kTK * KROW;
    static constexpr int LDS_V = DL * VROW;
};

// bf16 element c (0..7) of a 16-byte piece, widened to float
__device__ inline float bf16_at(const u32x4& d, int c) {
    const uint32_t w = d[c >> 1];
    return __uint_as_float((c & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

__device__ inline uint32_t pack_f16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

template <int NH, int DL, int DR>
struct Attend {
    using C = AttnShape<NH, DL, DR>;

    // Attend one query over selected rows sel[t_begin .. t_end) of a cache
    // holding nkeys rows.  Leaves, per lane, the unnormalised output for head
    // 16w + (lane & 15) and features 16fb + 4(lane >> 4) + i, the running
    // maximum m2 (log2 units) and the lane's share of the exponent sum.
    __device__ static void run(const uint16_t* __restrict__ qrow, const uint16_t* __restrict__ kv,
                               const int32_t* __restrict__ sel, int t_begin, int t_end, int nkeys,
                               float scale_log2, unsigned char* lds_k, unsigned char* lds_v,
                               uint32_t* lds_mask, f32x4 (&o)[C::FB], float& m2, float& lsum) {
        const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;
        const int head = 16 * w + c16;
        const u32x4 zero = {0u, 0u, 0u, 0u};

        u32x4 qf[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const int f = 32 * ks + 8 * g;
            qf[ks] = (head < NH && f < C::DQK) ? ldg16(qrow + (int64_t)head * C::DQK + f) : zero;
        }
#pragma unroll
        for (int fb = 0; fb < C::FB; ++fb) o[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
        m2 = -INFINITY;
        lsum = 0.f;

        if constexpr (C::DQKP > C::DQK) {   // K-dim padding columns stay zero
            constexpr int PP = (C::DQKP - C::DQK) / 8;
            for (int e = tid; e < kTK * PP; e += C::NT)
                *reinterpret_cast<u32x4*>(lds_k + (e / PP) * C::KROW + 2 * C::DQK + 16 * (e % PP)) = zero;
        }

        for (int t0 = t_begin; t0 < t_end; t0 += kTK) {
            // ---- gather the tile: latent part as 8x8 blocks, transposed copy in fp16
            constexpr int FO = DL / 8;
            for (int bi = tid; bi < 4 * FO; bi += C::NT) {
                const int ko = bi & 3, fo = bi >> 2;
                // key k of the tile sits at 8((k%16)/4) + 4(k/16) + k%4 in a value row:
                // keys 8ko+0..3 at pa.., keys 8ko+4..7 at pa+8..
                const int pa = 16 * (ko & 1) + 4 * (ko >> 1);
#pragma unroll
                for (int hv = 0; hv < 2; ++hv) {
                    u32x4 d[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = t0 + 8 * ko + 4 * hv + r;
                        const int j = sel[min(t, t_end - 1)];
                        const bool ok = t < t_end && (unsigned)j < (unsigned)nkeys;
                        d[r] = ldg16(kv + (int64_t)(ok ? j : 0) * C::DQK + 8 * fo);   // row 0 always exists
                        if (!ok) d[r] = zero;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        *reinterpret_cast<u32x4*>(lds_k + (8 * ko + 4 * hv + r) * C::KROW + 16 * fo) = d[r];
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        u32x2 v;
                        v[0] = pack_f16(bf16_at(d[0], c), bf16_at(d[1], c));
                        v[1] = pack_f16(bf16_at(d[2], c), bf16_at(d[3], c));
                        *reinterpret_cast<u32x2*>(lds_v + (8 * fo + c) * C::VROW + 2 * (pa + 8 * hv)) = v;
                    }
                }
            }
            constexpr int RO = DR / 8;
            for (int ci = tid; ci < kTK * RO; ci += C::NT) {
                const int key = ci / RO, part = ci % RO;
                const int t = t0 + key;
                const int j = sel[min(t, t_end - 1)];
                const bool ok = t < t_end && (unsigned)j < (unsigned)nkeys;
                u32x4 d = ldg16(kv + (int64_t)(ok ? j : 0) * C::DQK + DL + 8 * part);
                if (!ok) d = zero;
                *reinterpret_cast<u32x4*>(lds_k + key * C::KROW + 2 * DL + 16 * part) = d;
            }
            if (tid < 64) {
                const int t = t0 + tid;
                const int j = sel[min(t, t_end - 1)];
                const uint64_t bm = __ballot(tid < kTK && t < t_end && (unsigned)j < (unsigned)nkeys);
                if (tid == 0) *lds_mask = (uint32_t)bm;
            }
            __syncthreads();

            // ---- scores: S^T[key][head] for keys 0-15 (s0) and 16-31 (s1)
            const uint32_t vmask = *lds_mask;
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const u32x4 a0 = *reinterpret_cast<const u32x4*>(lds_k + c16 * C::KROW + 64 * ks + 16 * g);
                const u32x4 a1 = *reinterpret_cast<const u32x4*>(lds_k + (16 + c16) * C::KROW + 64 * ks + 16 * g);
                s0 = mfma16_bf16(a0, qf[ks], s0);
                s1 = mfma16_bf16(a1, qf[ks], s1);
            }
            // lane (g, c16) holds keys 4g+i (s0) and 16+4g+i (s1) of head c16
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = ((vmask >> (4 * g + i)) & 1u) ? s0[i] * scale_log2 : -INFINITY;
                x[4 + i] = ((vmask >> (16 + 4 * g + i)) & 1u) ? s1[i] * scale_log2 : -INFINITY;
            }
            float mx = x[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mnew = fmaxf(m2, mx);
            // all keys so far masked: keep the state at zero without NaNs
            const float mref = (mnew == -INFINITY) ? 0.f : mnew;
            const float alpha = exp2f(m2 - mref);
            float p[8], ps = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) { p[i] = exp2f(x[i] - mref); ps += p[i]; }
            lsum = lsum * alpha + ps;
            if (__ballot(alpha != 1.f)) {   // wave-uniform: skip when no maximum moved
#pragma unroll
                for (int fb = 0; fb < C::FB; ++fb) o[fb] *= alpha;
            }
            m2 = mnew;
            u32x4 pb;
            pb[0] = pack_f16(p[0], p[1]);
            pb[1] = pack_f16(p[2], p[3]);
            pb[2] = pack_f16(p[4], p[5]);
            pb[3] = pack_f16(p[6], p[7]);
            // ---- values: O^T[feature][head] += V^T[feature][keys] P^T[keys][head]
#pragma unroll
            for (int fb = 0; fb < C::FB; ++fb) {
                const u32x4 av = *reinterpret_cast<const u32x4*>(lds_v + (16 * fb + c16) * C::VROW + 16 * g);
                o[fb] = mfma16_f16(av, pb, o[fb]);
            }
            __syncthreads();
        }
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
    }
};

template <int NH, int DL, int DR>
__global__ __launch_bounds__((AttnShape<NH, DL, DR>::NT)) __attribute__((amdgpu_waves_per_eu(2)))
void attention_kernel(AttnArgs a) {
    using C = AttnShape<NH, DL, DR>;
    __shared__ __attribute__((aligned(16))) unsigned char lds_k[C::LDS_K];
    __shared__ __attribute__((aligned(16))) unsigned char lds_v[C::LDS_V];
    __shared__ uint32_t lds_mask;
    const int row = blockIdx.x;
    const int cnt = min(max(a.count[row], 0), a.top_k);
    f32x4 o[C::FB];
    float m2, lsum;
    Attend<NH, DL, DR>::run(a.q + (int64_t)row * NH * C::DQK, a.kv, a.idx + (int64_t)row * a.top_k, 0, cnt,
                            a.N, a.scale_log2, lds_k, lds_v, &lds_mask, o, m2, lsum);
    const int l = threadIdx.x & 63, g = l >> 4;
    const int head = 16 * (threadIdx.x >> 6) + (l & 15);
    if (head >= NH) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float* orow = a.out + ((int64_t)row * NH + head) * DL;
#pragma unroll
    for (int fb = 0; fb < C::FB; ++fb) *reinterpret_cast<f32x4*>(orow + 16 * fb + 4 * g) = o[fb] * inv;
    if (a.lse && g == 0)
        a.lse[(int64_t)row * NH + head] = lsum > 0.f ? (m2 + log2f(lsum)) * 0.69314718055994531f : -INFINITY;
}

template <int NH, int DL, int DR>
__global__ __launch_bounds__((AttnShape<NH, DL, DR>::NT)) __attribute__((amdgpu_waves_per_eu(2)))
void attention_split_kernel(AttnSplitArgs a, SeqMeta m) {
    using C = AttnShape<NH, DL, DR>;
    __shared__ __attribute__((aligned(16))) unsigned char lds_k[C::LDS_K];
    __shared__ __attribute__((aligned(16))) unsigned char lds_v[C::LDS_V];
    __shared__ uint32_t lds_mask;
    const int item = blockIdx.x;
    const int b = seq_of_block(m, item);
    const int ctx = m.ctx[b];
    const int cnt = min(ctx, a.top_k);
    const int t_begin = (item - m.blk0[b]) * a.chunk;
    const int t_end = min(t_begin + a.chunk, cnt);
    f32x4 o[C::FB];
    float m2, lsum;
    Attend<NH, DL, DR>::run(a.q + (int64_t)b * NH * C::DQK, a.kv + m.key_off[b] * C::DQK,
                            a.idx + (int64_t)b * a.top_k, t_begin, t_end, ctx, a.scale_log2, lds_k, lds_v,
                            &lds_mask, o, m2, lsum);
    const int l = threadIdx.x & 63, g = l >> 4;
    const int head = 16 * (threadIdx.x >> 6) + (l & 15);
    if (head >= NH) return;
    float* orow = a.part_o + ((int64_t)item * NH + head) * DL;
#pragma unroll
    for (int fb = 0; fb < C::FB; ++fb) *reinterpret_cast<f32x4*>(orow + 16 * fb + 4 * g) = o[fb];
    if (g == 0) {
        a.part_ml[((int64_t)item * NH + head) * 2 + 0] = m2;
        a.part_ml[((int64_t)item * NH + head) * 2 + 1] = lsum;
    }
}

// out[b,h,:] = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c over the chunks of b
template <int NH, int DL>
__global__ __launch_bounds__(128) void combine_kernel(AttnSplitArgs a, SeqMeta m) {
    const int b = blockIdx.x / NH, h = blockIdx.x % NH;
    const int it0 = m.blk0[b], it1 = m.blk0[b + 1];
    float M = -INFINITY;
    for (int it = it0; it < it1; ++it) M = fmaxf(M, a.part_ml[((int64_t)it * NH + h) * 2]);
    float den = 0.f;
    for (int it = it0; it < it1; ++it) {
        const float mi = a.part_ml[((int64_t)it * NH + h) * 2];
        if (mi != -INFINITY) den += exp2f(mi - M) * a.part_ml[((int64_t)it * NH + h) * 2 + 1];
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int f = 4 * threadIdx.x; f < DL; f += 4 * 128) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int it = it0; it < it1; ++it) {
            const float mi = a.part_ml[((int64_t)it * NH + h) * 2];
            if (mi == -INFINITY) continue;
            acc += exp2f(mi - M) * *reinterpret_cast<const f32x4*>(a.part_o + ((int64_t)it * NH + h) * DL + f);
        }
        *reinterpret_cast<f32x4*>(a.out + ((int64_t)b * NH + h) * DL + f) = acc * inv;
    }
}

}  // namespace

hipError_t launch_attention(int shape_id, const AttnArgs& a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    if (shape_id == 0)
        hipLaunchKernelGGL((attention_kernel<64, 512, 64>), dim3(a.rows), dim3(AttnShape<64, 512, 64>::NT), 0, s, a);
    else
        hipLaunchKernelGGL((attention_kernel<4, 64, 16>), dim3(a.rows), dim3(AttnShape<4, 64, 16>::NT), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_attention_split(int shape_id, const AttnSplitArgs& a, const SeqMeta& m, int items,
                                  hipStream_t s) {
    if (items <= 0) return hipSuccess;
    if (shape_id == 0) {
        hipLaunchKernelGGL((attention_split_kernel<64, 512, 64>), dim3(items), dim3(AttnShape<64, 512, 64>::NT), 0,
                           s, a, m);
        hipLaunchKernelGGL((combine_kernel<64, 512>), dim3(m.B * 64), dim3(128), 0, s, a, m);
    } else {
        hipLaunchKernelGGL((attention_split_kernel<4, 64, 16>), dim3(items), dim3(AttnShape<4, 64, 16>::NT), 0, s,
                           a, m);
        hipLaunchKernelGGL((combine_kernel<4, 64>), dim3(m.B * 4), dim3(128), 0, s, a, m);
    }
    return hipGetLastError();
}

}  // namespace dsa
