// topk.hip - per-query top-k selection over indexer scores on gfx950.
//
// exo PR #2539, Prefill section: each query keeps its index_topk (2048)
// best-scoring causal keys; a query with no more causal keys than that keeps
// every earlier key.  Readings: ties go to the lower key index; the kept keys
// are written in ascending key order and padded with -1.
//
// Design: one 1024-thread block per query row.  The row's scores live in
// VGPRs (EPT per thread, element e of thread t is key e*1024 + t, so loads
// are coalesced) as order-preserving uint32 keys.  Four 8-bit radix passes
// over an LDS histogram find T, the top_k-th largest key, and how many keys
// equal to T must be kept.  Then every kept key's output slot is the number
// of kept keys with a lower index: ballot bit counts per (element, wave)
// plus one block-wide exclusive scan, so the output comes out in ascending
// key order with no sort.  Every step is integer work: the result is exact.
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Larger float -> larger key; -0 ranks equal to +0 (the floats compare equal).
__device__ inline uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct TopkSmem {
    int hist[256];
    int sel_bin;
    int sel_krem;
    int pre_gt[kTopkThreads];
    int pre_eq[kTopkThreads];
    int wsum_gt[kTopkWaves];
    int wsum_eq[kTopkWaves];
};

__device__ inline uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

// Block-wide exclusive scan of (a, b) held one pair per thread.
__device__ inline void block_exclusive_scan2(int& a, int& b, TopkSmem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int ia = a, ib = b;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int ya = __shfl_up(ia, d), yb = __shfl_up(ib, d);
        if (lane >= d) { ia += ya; ib += yb; }
    }
    if (lane == 63) { sm.wsum_gt[wave] = ia; sm.wsum_eq[wave] = ib; }
    __syncthreads();
    int oa = 0, ob = 0;
    for (int v = 0; v < wave; ++v) { oa += sm.wsum_gt[v]; ob += sm.wsum_eq[v]; }
    a = oa + ia - a;
    b = ob + ib - b;
}

template <int EPT>
__device__ void topk_row(const float* __restrict__ srow, int n, int top_k, int32_t* __restrict__ out,
                         int32_t* count, TopkSmem& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (n <= top_k) {   // every earlier key; the scores are not read
        for (int t = tid; t < top_k; t += kTopkThreads) out[t] = t < n ? t : -1;
        if (tid == 0 && count) *count = n;
        return;
    }
    uint32_t u[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int gi = e * kTopkThreads + tid;
        u[e] = gi < n ? order_key(srow[gi]) : 0u;
    }

    // radix select: find the top_k-th largest key T, most significant byte first
    uint32_t prefix = 0, pmask = 0;
    int krem = top_k;
    for (int pass = 3; pass >= 0; --pass) {
        const int shift = pass * 8;
        if (tid < 256) sm.hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int gi = e * kTopkThreads + tid;
            if (gi < n && (u[e] & pmask) == prefix) atomicAdd(&sm.hist[(u[e] >> shift) & 255u], 1);
        }
        __syncthreads();
        if (wave == 0) {
            int h[4], tot = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) { h[k] = sm.hist[4 * lane + k]; tot += h[k]; }
            // keys in bins above this lane's four bins: suffix sum over higher lanes
            int suf = tot;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_down(suf, d);
                if (lane + d < 64) suf += y;
            }
            int gt = suf - tot;
#pragma unroll
            for (int k = 3; k >= 0; --k) {
                if (gt < krem && gt + h[k] >= krem) { sm.sel_bin = 4 * lane + k; sm.sel_krem = krem - gt; }
                gt += h[k];
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sm.sel_bin << shift;
        pmask |= 0xFFu << shift;
        krem = sm.sel_krem;
    }
    const uint32_t T = prefix;   // keep every key > T and the first krem keys == T

    // per (element, wave) counts of keys > T and == T
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int gi = e * kTopkThreads + tid;
        const uint64_t gm = __ballot(gi < n && u[e] > T);
        const uint64_t qm = __ballot(gi < n && u[e] == T);
        if (lane == 0) { sm.pre_gt[e * kTopkWaves + wave] = __popcll(gm); sm.pre_eq[e * kTopkWaves + wave] = __popcll(qm); }
    }
    __syncthreads();
    int a = 0, b = 0;
    if (tid < EPT * kTopkWaves) { a = sm.pre_gt[tid]; b = sm.pre_eq[tid]; }
    block_exclusive_scan2(a, b, sm);
    __syncthreads();
    if (tid < EPT * kTopkWaves) { sm.pre_gt[tid] = a; sm.pre_eq[tid] = b; }
    __syncthreads();

    const uint64_t lt = lanemask_lt(lane);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int gi = e * kTopkThreads + tid;
        const bool g = gi < n && u[e] > T;
        const bool q = gi < n && u[e] == T;
        const uint64_t gm = __ballot(g), qm = __ballot(q);
        const int gt_before = sm.pre_gt[e * kTopkWaves + wave] + __popcll(gm & lt);
        const int eq_before = sm.pre_eq[e * kTopkWaves + wave] + __popcll(qm & lt);
        // slots are < top_k by construction; the bound only guards the store
        const int slot = g ? gt_before + min(eq_before, krem) : gt_before + eq_before;
        if ((g || (q && eq_before < krem)) && slot < top_k) out[slot] = gi;
    }
    if (tid == 0 && count) *count = top_k;
}

template <int EPT>
__global__ __launch_bounds__(kTopkThreads) void topk_prefill_kernel(TopkArgs a) {
    __shared__ TopkSmem sm;
    const int r = blockIdx.x;
    const int64_t p = a.pos0 + r;
    const int n = (int)(p + 1);
    const float* srow = (n > a.top_k) ? a.S + (int64_t)(r - a.s_row0) * a.ldS : nullptr;
    topk_row<EPT>(srow, n, a.top_k, a.idx + (int64_t)r * a.top_k, a.count ? a.count + r : nullptr, sm);
}

template <int EPT>
__global__ __launch_bounds__(kTopkThreads) void topk_decode_kernel(const float* S, SeqMeta m, int top_k,
                                                                  int32_t* idx, int32_t* count) {
    __shared__ TopkSmem sm;
    const int b = blockIdx.x;
    topk_row<EPT>(S + m.s_off[b], m.ctx[b], top_k, idx + (int64_t)b * top_k, count ? count + b : nullptr, sm);
}

int ept_for(int n_max) {
    int e = 2;
    while (e * kTopkThreads < n_max) e *= 2;
    return e;
}

}  // namespace

hipError_t launch_topk_prefill(const TopkArgs& a, int n_max, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    dim3 grid(a.rows), block(kTopkThreads);
    switch (ept_for(n_max)) {
        case 2: hipLaunchKernelGGL(topk_prefill_kernel<2>, grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL(topk_prefill_kernel<4>, grid, block, 0, s, a); break;
        case 8: hipLaunchKernelGGL(topk_prefill_kernel<8>, grid, block, 0, s, a); break;
        case 16: hipLaunchKernelGGL(topk_prefill_kernel<16>, grid, block, 0, s, a); break;
        case 32: hipLaunchKernelGGL(topk_prefill_kernel<32>, grid, block, 0, s, a); break;
        case 64: hipLaunchKernelGGL(topk_prefill_kernel<64>, grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_topk_decode(const float* S, const SeqMeta& m, int top_k, int32_t* idx,
                              int32_t* count, int n_max, hipStream_t s) {
    if (m.B <= 0) return hipSuccess;
    dim3 grid(m.B), block(kTopkThreads);
    switch (ept_for(n_max)) {
        case 2: hipLaunchKernelGGL(topk_decode_kernel<2>, grid, block, 0, s, S, m, top_k, idx, count); break;
        case 4: hipLaunchKernelGGL(topk_decode_kernel<4>, grid, block, 0, s, S, m, top_k, idx, count); break;
        case 8: hipLaunchKernelGGL(topk_decode_kernel<8>, grid, block, 0, s, S, m, top_k, idx, count); break;
        case 16: hipLaunchKernelGGL(topk_decode_kernel<16>, grid, block, 0, s, S, m, top_k, idx, count); break;
        case 32: hipLaunchKernelGGL(topk_decode_kernel<32>, grid, block, 0, s, S, m, top_k, idx, count); break;
        case 64: hipLaunchKernelGGL(topk_decode_kernel<64>, grid, block, 0, s, S, m, top_k, idx, count); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dsa
