// router.hip - MoE router selection on gfx950.
//
// "GLM-5.2-Vision: llama.cpp vs vLLM line-by-line pipeline trace", section 8a
// (Gating), and exo PR #2539 (router selection in one kernel): per token the
// expert probabilities are the sigmoid of the float32 router logits; the
// per-expert bias is added for the choice only; the k best experts are kept;
// their weights are the unbiased probabilities over their sum, the sum
// clamped below at 6.1e-5, times the routed scaling factor (GLM: 256
// experts, 8 per token, factor 2.5, one expert group, so no group masking).
//
// One wave per token, 64 / E of the experts per lane (strided so every load
// is coalesced).  A probability is the exact sigmoid rounded once to float
// (evaluated in double), the selection score is that float plus the bias in
// float arithmetic, and each selection key packs the order-preserving bits
// of the score above the complemented expert index, so one 64-bit maximum
// picks the highest score and, among equal scores, the lowest index.  The
// k rounds each take a wave maximum in registers (DPP and lane-swap moves)
// and retire the winner.
// Weights are formed in double in selection order and rounded to float.
#include "dsa_kernels.h"

#include <math.h>

namespace dsa {
namespace {

constexpr int kRouterThreads = 256;
constexpr double kWeightSumMin = 6.1e-5;

__device__ inline uint32_t orderable(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// v from the lane a DPP pattern names (both halves moved the same way)
template <int CTRL>
__device__ inline uint64_t dpp64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}

// Maximum over the wave, in every lane, without LDS: within each row of 16
// lanes by DPP (swap neighbours, swap pairs, rotate the row by 4 and by 8),
// then across rows with v_permlane16_swap / v_permlane32_swap.
__device__ inline uint64_t wave_max_u64(uint64_t v) {
    v = umax64(v, dpp64<0xB1>(v));    // quad_perm [1,0,3,2]
    v = umax64(v, dpp64<0x4E>(v));    // quad_perm [2,3,0,1]
    v = umax64(v, dpp64<0x124>(v));   // row_ror:4
    v = umax64(v, dpp64<0x128>(v));   // row_ror:8
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    v = umax64(((uint64_t)b[0] << 32) | a[0], ((uint64_t)b[1] << 32) | a[1]);
    lo = (uint32_t)v;
    hi = (uint32_t)(v >> 32);
    a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    return umax64(((uint64_t)b[0] << 32) | a[0], ((uint64_t)b[1] << 32) | a[1]);
}

template <int EPL>
__global__ __launch_bounds__(kRouterThreads) void router_topk_kernel(RouterArgs a) {
    constexpr int E = 64 * EPL;
    const int t = (int)((blockIdx.x * kRouterThreads + threadIdx.x) >> 6);
    const int l = threadIdx.x & 63;
    if (t >= a.T) return;   // whole waves only
    const float* lg = a.logits + (int64_t)t * E;
    float p[EPL];
    uint64_t key[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = 64 * j + l;
        p[j] = (float)(1.0 / (1.0 + exp(-(double)lg[e])));
        const float s = p[j] + a.bias[e];
        key[j] = ((uint64_t)orderable(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
    }
    // k rounds: wave maximum, then the owner retires the winner; lane r keeps
    // the r-th expert and its probability
    int my_e = 0;
    float my_p = 0.f;
    double sum = 0.0;
    for (int r = 0; r < a.k; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
        best = wave_max_u64(best);
        const int e = __builtin_amdgcn_readfirstlane((int)(0xFFFFFFFFu - (uint32_t)best));
        const int owner = e & 63, jw = e >> 6;
        float pw = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            if (j == jw) {
                pw = p[j];
                if (l == owner) key[j] = 0;
            }
        }
        pw = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(pw), owner));
        sum += (double)pw;
        if (l == r) { my_e = e; my_p = pw; }
    }
    if (l < a.k) {
        const double den = sum > kWeightSumMin ? sum : kWeightSumMin;
        a.ids[(int64_t)t * a.k + l] = my_e;
        a.weights[(int64_t)t * a.k + l] = (float)((double)my_p / den * (double)a.scale);
    }
}

}  // namespace

hipError_t launch_router_topk(const RouterArgs& a, hipStream_t s) {
    if (a.T <= 0) return hipSuccess;
    const int64_t threads = (int64_t)a.T * 64;
    const dim3 grid((unsigned)((threads + kRouterThreads - 1) / kRouterThreads)), block(kRouterThreads);
    switch (a.E) {
        case 64: hipLaunchKernelGGL(router_topk_kernel<1>, grid, block, 0, s, a); break;
        case 128: hipLaunchKernelGGL(router_topk_kernel<2>, grid, block, 0, s, a); break;
        case 256: hipLaunchKernelGGL(router_topk_kernel<4>, grid, block, 0, s, a); break;
        case 512: hipLaunchKernelGGL(router_topk_kernel<8>, grid, block, 0, s, a); break;
        case 1024: hipLaunchKernelGGL(router_topk_kernel<16>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dsa
