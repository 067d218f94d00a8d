// topk.hip - per-query top-k selection over indexer scores on gfx950.
//
// exo PR #2539, Prefill section: each query keeps its index_topk (2048)
// best-scoring causal keys; a query with no more causal keys than that keeps
// every earlier key.  Readings: ties go to the lower key index; the kept keys
// are written in ascending key order and padded with -1.
//
// Design: one block per query row; the row's scores stay in VGPRs (EPT per
// thread, element e of thread t is key e*NT + t, so loads are coalesced) as
// order-preserving uint32 keys.  The selection only needs T, the top_k-th
// largest key, and krem, how many keys equal to T are kept:
//   1. Value-linear histogram levels.  Live keys ("alive": every key the
//      levels so far have not ruled out) are binned by a monotone map of
//      their float value onto [0, 256) between the live minimum and maximum.
//      The bin holding the top_k-th key stays alive; bins above it are kept,
//      bins below are dropped.  Bins that follow the value (not the float's
//      exponent bits) spread a bell-shaped score row over many LDS counters,
//      so the atomics rarely collide.
//   2. Once at most NT keys are alive they are ranked directly (each thread
//      counts the live keys above its own), which yields T exactly.
//   3. Degenerate rows (non-finite values, a value range too wide or too
//      narrow for fp32 binning, too many levels) finish with an exact
//      32-step bisection over the live keys.  Every loop is bounded.
// Finally every kept key's output slot is the number of kept keys with a
// lower index (ballot counts per (element, wave) plus one block-wide scan),
// so the output is in ascending key order with no sort.  Every decision is
// taken on integer keys: the result is exact.
#include "dsa_kernels.h"

#include <type_traits>

namespace dsa {
namespace {

constexpr int kBins = 256;
constexpr int kMaxLevels = 4;
constexpr int kDecodeSeg = 16384;   // keys per decode segment block (a 64k context: 4 segments, 8192 candidates)

// Larger float -> larger key; -0 ranks equal to +0 (the floats compare equal).
__device__ inline uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key (up to the -0 merge).
__device__ inline float key_value(uint32_t k) {
    const uint32_t t = (uint32_t)((int32_t)k >> 31);     // all ones for keys of non-negative floats
    return __uint_as_float(~(k ^ (t & 0x7FFFFFFFu)));
}

// number of set bits of m in the lanes below this one
__device__ inline int count_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int NT, int EPT>
struct TopkSmem {
    static constexpr int NW = NT / 64;
    float red[2][2][NW];             // min / max partials, double buffered
    int cnt[2][NW];                  // bisection counts, double buffered
    int hist[kBins];
    float cand[NT];
    int ncand;
    int bstar, above, inbin;
    float T;
    int keep;
    int pre_gt[EPT * NW];
    int pre_eq[EPT * NW];
    int wsum_gt[NW];
    int wsum_eq[NW];
};

// Block-wide exclusive scan of (a, b) held one pair per thread.
template <int NT, int EPT>
__device__ inline void block_exclusive_scan2(int& a, int& b, TopkSmem<NT, EPT>& sm) {
    constexpr int NW = NT / 64;
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
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        if (v < wave) { oa += sm.wsum_gt[v]; ob += sm.wsum_eq[v]; }
    }
    a = oa + ia - a;
    b = ob + ib - b;
}

// Block-wide minimum and maximum (every thread gets both).
template <int NT, int EPT>
__device__ inline void block_minmax(float& lo, float& hi, int& par, TopkSmem<NT, EPT>& sm) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, d));
        hi = fmaxf(hi, __shfl_xor(hi, d));
    }
    if (lane == 0) { sm.red[par][0][wave] = lo; sm.red[par][1][wave] = hi; }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < NW; ++v) { lo = fminf(lo, sm.red[par][0][v]); hi = fmaxf(hi, sm.red[par][1][v]); }
    lo = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, lo)));
    hi = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, hi)));
    par ^= 1;
}

// The bin of a live value: trunc((v - lo) * scale) clamped to [0, 255].  A
// non-decreasing function of v (each rounding is monotone), so higher bins
// hold larger values and equal values share a bin.
__device__ inline int value_bin(float v, float lo, float scale) {
    const int b = (int)((v - lo) * scale);
    return min(max(b, 0), kBins - 1);
}

// Element k of a row: its score, and the key index written for it.
struct DirectRow {   // element k is key k
    static constexpr bool kRemap = false;
    const float* __restrict__ s;
    __device__ __forceinline__ float load(int k) const { return s[k]; }
    __device__ __forceinline__ int32_t index(int k) const { return k; }
};
// The candidates of a segmented row: the concatenated selections of its
// segments (seg keys each, top_k entries per segment, each in ascending
// order and padded with -1), so element order is key order.  An entry holds
// a key index local to its segment.  Padding entries score -inf; they are
// never kept, because every full segment brings top_k finite scores.
struct CandRow {
    static constexpr bool kRemap = true;   // outputs are element positions until remapped
    const float* __restrict__ s;       // the sequence's scores
    const int32_t* __restrict__ cand;
    int top_k, seg;
    __device__ __forceinline__ int32_t key(int k) const {
        const int c = cand[k];
        return c < 0 ? -1 : (k / top_k) * seg + c;
    }
    __device__ __forceinline__ float load(int k) const {
        const int j = key(k);
        return j < 0 ? -INFINITY : s[j];
    }
    __device__ __forceinline__ int32_t index(int k) const { return key(k); }
};

template <int NT, int EPT, typename Row>
__device__ __forceinline__ void topk_row(const Row& row, int n, int top_k,
                                         int32_t* __restrict__ out, int32_t* count, TopkSmem<NT, EPT>& sm) {
    static_assert(NT >= kBins && NT % 64 == 0 && EPT >= 1 && EPT <= 64, "topk geometry");
    static_assert(EPT * (NT / 64) <= NT, "one scan slot per thread");
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (n <= top_k) {   // every earlier key; the scores are not read
        for (int t = tid; t < top_k; t += NT) out[t] = t < n ? t : -1;
        if (tid == 0 && count) *count = n;
        return;
    }
    // Scores in registers.  A NaN score ranks as -inf; keys past the row are
    // NaN, which every comparison below treats as "not a candidate".
    const float kNone = __int_as_float(0x7FC00000);
    float f[EPT];
    const int nfull = n / NT;     // elements every lane of the block holds
#pragma unroll
    for (int e = 0; e < EPT; ++e)   // every load in bounds; no waits between them
        f[e] = row.load(e < nfull ? e * NT + tid : min(e * NT + tid, n - 1));
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const float x = f[e] == f[e] ? f[e] : -INFINITY;
        f[e] = e * NT + tid < n ? x : kNone;
    }
    if (tid == 0) { sm.ncand = 0; sm.T = INFINITY; sm.keep = 0; }
    if (tid < kBins) sm.hist[tid] = 0;

    // the live set is every key with lo <= value <= hi; krem of them are kept
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPT; ++e) { lo = fminf(lo, f[e]); hi = fmaxf(hi, f[e]); }
    int par = 0;
    block_minmax<NT, EPT>(lo, hi, par, sm);
    int krem = top_k;
    bool found = false;
    float T = 0.f;

    for (int lev = 0; lev < kMaxLevels; ++lev) {
        if (!(lo < hi)) { T = lo; found = true; break; }   // every live value equal (-0 == +0)
        const float scale = (float)kBins / (hi - lo);
        // finite positive scale only (excludes infinities and overflowing ranges)
        if (!(scale > 0.f && scale < 3.0e38f)) break;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const bool live = f[e] >= lo && f[e] <= hi;
            if (__ballot(live)) {
                if (live) atomicAdd(&sm.hist[value_bin(f[e], lo, scale)], 1);
            }
        }
        __syncthreads();
        if (wave == 0) {
            // bins 4*lane .. 4*lane+3; keys in higher bins come from higher lanes
            int h[4], tot = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) { h[k] = sm.hist[4 * lane + k]; tot += h[k]; }
            int suf = tot;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_down(suf, d);
                if (lane + d < 64) suf += y;
            }
            int gt = suf - tot;
#pragma unroll
            for (int k = 3; k >= 0; --k) {
                if (gt < krem && gt + h[k] >= krem) { sm.bstar = 4 * lane + k; sm.above = gt; sm.inbin = h[k]; }
                gt += h[k];
            }
        }
        __syncthreads();
        // recompute bins below rather than keep EPT of them (and EPT lane
        // masks) alive across the barrier
#pragma unroll
        for (int e = 0; e < EPT; ++e) asm volatile("" : "+v"(f[e]));
        const int bstar = __builtin_amdgcn_readfirstlane(sm.bstar);
        const int inbin = __builtin_amdgcn_readfirstlane(sm.inbin);
        krem -= __builtin_amdgcn_readfirstlane(sm.above);
        if (inbin <= NT) {
            // rank the keys of the bin directly: gather them, then each thread
            // counts the gathered values above and at its own
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const bool a = f[e] >= lo && f[e] <= hi && value_bin(f[e], lo, scale) == bstar;
                const uint64_t m = __ballot(a);
                if (m) {
                    int base = 0;
                    if (lane == 0) base = atomicAdd(&sm.ncand, __popcll(m));
                    base = __shfl(base, 0);
                    const int slot = base + count_below(m);
                    if (a && slot < NT) sm.cand[slot] = f[e];
                }
            }
            __syncthreads();
            // each key of the bin is ranked by P lanes (a power of two, up to
            // 16), which split the comparisons and combine them by shuffles
            int lg = 0;
            while (lg < 4 && (inbin << (lg + 1)) <= NT) ++lg;
            const int P = 1 << lg;
            const int c = tid >> lg, part = tid & (P - 1);
            int gt = 0, ge = 0;
            const float v = sm.cand[min(c, max(inbin - 1, 0))];
            if (c < inbin) {
#pragma unroll 4
                for (int i = part; i < inbin; i += P) {
                    const float x = sm.cand[i];
                    gt += x > v;
                    ge += x >= v;
                }
            }
            for (int d = 1; d < P; d <<= 1) {
                gt += __shfl_xor(gt, d);
                ge += __shfl_xor(ge, d);
            }
            if (c < inbin && part == 0 && gt < krem && krem <= ge) { sm.T = v; sm.keep = krem - gt; }
            __syncthreads();
            T = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sm.T)));
            krem = __builtin_amdgcn_readfirstlane(sm.keep);
            found = true;
            break;
        }
        // narrow the live range to the bin's values
        float nlo = INFINITY, nhi = -INFINITY;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const bool a = f[e] >= lo && f[e] <= hi && value_bin(f[e], lo, scale) == bstar;
            nlo = a ? fminf(nlo, f[e]) : nlo;
            nhi = a ? fmaxf(nhi, f[e]) : nhi;
        }
        if (tid < kBins) sm.hist[tid] = 0;
        lo = nlo;
        hi = nhi;
        block_minmax<NT, EPT>(lo, hi, par, sm);
    }

    if (!found) {
        // exact bisection on order-preserving keys: the largest key t with
        // #(live keys >= t) >= krem, then the live keys above t are kept
        uint32_t t = 0;
#pragma unroll 1
        for (int bit = 31; bit >= -1; --bit) {
            const uint32_t c = bit >= 0 ? (t | (1u << bit)) : t + 1u;
            int w = 0;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                asm volatile("" : "+v"(f[e]));   // recompute per step: no hoisted masks or keys
                w += (f[e] >= lo && f[e] <= hi && order_key(f[e]) >= c) ? 1 : 0;
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) w += __shfl_xor(w, d);
            if (lane == 0) sm.cnt[par][wave] = w;
            __syncthreads();
            int tot = 0;
#pragma unroll
            for (int v = 0; v < NW; ++v) tot += sm.cnt[par][v];
            tot = __builtin_amdgcn_readfirstlane(tot);
            par ^= 1;
            if (bit >= 0) {
                if (tot >= krem) t = c;
            } else {
                krem -= (t == 0xFFFFFFFFu) ? 0 : tot;
            }
        }
        T = key_value(t);
    }
    // keep every key > T and the first krem keys == T (NaN padding is neither)
    const int keep = krem;

    // per (element, wave) counts of keys > T and == T; lane e of each wave
    // collects element e's counts
    int cg = 0, cq = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int ng = __popcll(__ballot(f[e] > T));
        const int nq = __popcll(__ballot(f[e] == T));
        cg = (lane == e) ? ng : cg;
        cq = (lane == e) ? nq : cq;
    }
    if (lane < EPT) { sm.pre_gt[lane * NW + wave] = cg; sm.pre_eq[lane * NW + wave] = cq; }
    __syncthreads();
    int a = 0, b = 0;
    if (tid < EPT * NW) { a = sm.pre_gt[tid]; b = sm.pre_eq[tid]; }
    block_exclusive_scan2<NT, EPT>(a, b, sm);
    __syncthreads();
    if (tid < EPT * NW) { sm.pre_gt[tid] = a; sm.pre_eq[tid] = b; }
    __syncthreads();
    // lane e holds element e's exclusive counts (read back one per element)
    const int pg_l = lane < EPT ? sm.pre_gt[lane * NW + wave] : 0;
    const int pq_l = lane < EPT ? sm.pre_eq[lane * NW + wave] : 0;

#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        // one element at a time: keeps the compiler from computing all
        // 2*EPT lane masks up front (they would spill)
        asm volatile("" : "+v"(f[e]));
        int t_ = tid;                      // fresh copy: the key index is not kept from the loads
        asm volatile("" : "+v"(t_));
        const uint64_t gm = __ballot(f[e] > T);
        const uint64_t qm = __ballot(f[e] == T);
        if (gm | qm) {
            const int pg = __builtin_amdgcn_readlane(pg_l, e);
            const int pq = __builtin_amdgcn_readlane(pq_l, e);
            // the group's keys equal to T that are kept: the first (keep - pq)
            uint64_t qsel = 0;
            const int room = keep - pq;              // signed: negative once every tie is placed
            if (room >= (int)__popcll(qm)) {
                qsel = qm;
            } else if (room > 0) {
                uint64_t m = qm;
                for (int k = 0; k < room; ++k) { qsel |= m & (~m + 1); m &= m - 1; }
            }
            const uint64_t sel = gm | qsel;
            const int base = pg + min(pq, keep);    // kept keys in earlier groups
            const int slot = base + count_below(sel);
            if (((sel >> lane) & 1) && slot >= 0 && slot < top_k) out[slot] = e * NT + t_;
        }
    }
    if constexpr (Row::kRemap) {
        // element positions -> key indices, in one coalesced pass (a lookup
        // per kept element inside the loop above would serialise its loads)
        __syncthreads();
        for (int t = tid; t < top_k; t += NT) out[t] = row.index(out[t]);
    }
    if (tid == 0 && count) *count = top_k;
}

template <int NT, int EPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 8))) void topk_prefill_kernel(TopkArgs a) {
    __shared__ TopkSmem<NT, EPT> sm;
    const int r = blockIdx.x;
    const int64_t p = a.pos0 + r;
    const int n = (int)(p + 1);
    const float* srow = (n > a.top_k) ? a.S + (int64_t)(r - a.s_row0) * a.ldS : nullptr;
    topk_row<NT, EPT>(DirectRow{srow}, n, a.top_k, a.idx + (int64_t)r * a.top_k, a.count ? a.count + r : nullptr,
                      sm);
}

// Decode, phase 1: block -> (sequence b, segment g) of kDecodeSeg keys.  A
// sequence of one segment is finished here; otherwise the segment's
// selection goes to the candidate list (top_k entries per segment block).
template <int NT, int EPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 8))) void topk_decode_kernel(
        const float* S, SeqMeta m, int top_k, int32_t* idx, int32_t* count, int32_t* cand) {
    __shared__ TopkSmem<NT, EPT> sm;
    const int b = seq_of_block(m, blockIdx.x);
    const int g = blockIdx.x - m.blk0[b];
    const int ctx = m.ctx[b];
    const int k0 = g * kDecodeSeg;
    const int n = min(ctx - k0, kDecodeSeg);
    const float* srow = S + m.s_off[b] + k0;
    if (ctx <= kDecodeSeg)
        topk_row<NT, EPT>(DirectRow{srow}, n, top_k, idx + (int64_t)b * top_k, count ? count + b : nullptr, sm);
    else
        topk_row<NT, EPT>(DirectRow{srow}, n, top_k, cand + (int64_t)blockIdx.x * top_k, nullptr, sm);
}

// Decode, phase 2: block b selects sequence b's top_k among the candidates
// of its segments (sequences of one segment have nothing to do).
template <int NT, int EPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4, 8))) void topk_merge_kernel(
        const float* S, SeqMeta m, int top_k, int32_t* idx, int32_t* count, const int32_t* cand) {
    __shared__ TopkSmem<NT, EPT> sm;
    const int b = blockIdx.x;
    const int nseg = m.blk0[b + 1] - m.blk0[b];
    if (nseg < 2) return;
    const CandRow row{S + m.s_off[b], cand + (int64_t)m.blk0[b] * top_k, top_k, kDecodeSeg};
    topk_row<NT, EPT>(row, nseg * top_k, top_k, idx + (int64_t)b * top_k, count ? count + b : nullptr, sm);
}

// Block shape by row length: up to 32 keys per thread in 256-, then 512-,
// then 1024-thread blocks; 64 per thread only for the longest rows.  Short
// rows keep many blocks in flight per CU; every shape stays within 128 VGPRs.
template <typename Launch>
hipError_t dispatch_shape(int n_max, Launch&& launch) {
    using std::integral_constant;
    if (n_max <= 256) return launch(integral_constant<int, 256>{}, integral_constant<int, 1>{});
    if (n_max <= 512) return launch(integral_constant<int, 256>{}, integral_constant<int, 2>{});
    if (n_max <= 1024) return launch(integral_constant<int, 256>{}, integral_constant<int, 4>{});
    if (n_max <= 2048) return launch(integral_constant<int, 256>{}, integral_constant<int, 8>{});
    if (n_max <= 4096) return launch(integral_constant<int, 256>{}, integral_constant<int, 16>{});
    if (n_max <= 8192) return launch(integral_constant<int, 256>{}, integral_constant<int, 32>{});
    if (n_max <= 16384) return launch(integral_constant<int, 512>{}, integral_constant<int, 32>{});
    if (n_max <= 32768) return launch(integral_constant<int, 1024>{}, integral_constant<int, 32>{});
    if (n_max <= 65536) return launch(integral_constant<int, 1024>{}, integral_constant<int, 64>{});
    return hipErrorInvalidValue;
}

// Decode: one row per sequence, so latency rather than throughput counts:
// always 1024 threads, as few elements per thread as the row allows.
template <typename Launch>
hipError_t dispatch_wide(int n_max, Launch&& launch) {
    using std::integral_constant;
    if (n_max <= 1024) return launch(integral_constant<int, 1024>{}, integral_constant<int, 1>{});
    if (n_max <= 2048) return launch(integral_constant<int, 1024>{}, integral_constant<int, 2>{});
    if (n_max <= 4096) return launch(integral_constant<int, 1024>{}, integral_constant<int, 4>{});
    if (n_max <= 8192) return launch(integral_constant<int, 1024>{}, integral_constant<int, 8>{});
    // segments of kDecodeSeg keys, and at most 8 * kMaxTopK candidates
    static_assert(kDecodeSeg <= 16384 && (kMaxSelectKeys / kDecodeSeg) * kMaxTopK <= 16384, "decode shapes");
    if (n_max <= 16384) return launch(integral_constant<int, 1024>{}, integral_constant<int, 16>{});
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_topk_prefill(const TopkArgs& a, int n_max, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    return dispatch_shape(n_max, [&](auto nt, auto ept) {
        constexpr int NT = decltype(nt)::value, EPT = decltype(ept)::value;
        hipLaunchKernelGGL((topk_prefill_kernel<NT, EPT>), dim3(a.rows), dim3(NT), 0, s, a);
        return hipGetLastError();
    });
}

int topk_decode_segments(int ctx) { return (ctx + kDecodeSeg - 1) / kDecodeSeg; }

hipError_t launch_topk_decode(const float* S, const SeqMeta& m, int top_k, int32_t* idx, int32_t* count,
                              int32_t* cand, int n_max, hipStream_t s) {
    if (m.B <= 0) return hipSuccess;
    const int blocks = m.blk0[m.B];
    hipError_t e = dispatch_wide(min(n_max, kDecodeSeg), [&](auto nt, auto ept) {
        constexpr int NT = decltype(nt)::value, EPT = decltype(ept)::value;
        hipLaunchKernelGGL((topk_decode_kernel<NT, EPT>), dim3(blocks), dim3(NT), 0, s, S, m, top_k, idx, count, cand);
        return hipGetLastError();
    });
    if (e != hipSuccess || n_max <= kDecodeSeg) return e;
    return dispatch_wide(topk_decode_segments(n_max) * top_k, [&](auto nt, auto ept) {
        constexpr int NT = decltype(nt)::value, EPT = decltype(ept)::value;
        hipLaunchKernelGGL((topk_merge_kernel<NT, EPT>), dim3(m.B), dim3(NT), 0, s, S, m, top_k, idx, count, cand);
        return hipGetLastError();
    });
}

}  // namespace dsa
