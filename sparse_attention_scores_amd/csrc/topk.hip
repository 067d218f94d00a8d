// topk.hip - per-query top-k selection over indexer scores on gfx950.
//
// exo PR #2539, Prefill section: each query keeps its index_topk (2048)
// best-scoring causal keys; a query with no more causal keys than that keeps
// every earlier key.  Readings: ties go to the lower key index; the kept keys
// are written in ascending key order and padded with -1.
//
// Design: one block per query row; the row's scores stay in VGPRs (EPT per
// thread, element e of thread t is key e*NT + t, so loads are coalesced).
// The selection only needs T, the top_k-th largest score, and krem, how many
// keys equal to T are kept:
//   1. Value-linear histogram levels.  Live keys ("alive": every key the
//      levels so far have not ruled out) are binned by a monotone map of
//      their float value onto [0, 256) between the live minimum and maximum.
//      The bin holding the top_k-th key stays alive; bins above it are kept,
//      bins below are dropped.  Bins that follow the value (not the float's
//      exponent bits) spread a bell-shaped score row over many LDS counters,
//      so the atomics rarely collide.
//   2. Once at most NT keys are alive, one pass over the keys writes the
//      LDS bitmap of the keys above the boundary bin (bit k is element k:
//      each wave stores its 64-lane ballot masks) and gathers the bin's keys
//      (each wave into its own LDS slice).  The gathered keys are ranked
//      directly: each sets its bit when it is among the krem best, and the
//      keys equal to T, when only some of them fit, go to a tie bitmap.
//   3. Degenerate rows (non-finite values, a value range too wide or too
//      narrow for fp32 binning, too many levels) finish with an exact
//      32-step bisection over the live keys, then one pass writes the
//      bitmaps of the keys above T and equal to T.  Every loop is bounded.
// Finally each thread walks a few consecutive words of the bitmaps after one
// block-wide scan of their counts (keeping the lowest of the ties that
// fit), so the output is in ascending key order with no sort.  Every
// decision is an exact float comparison (-0 and +0 compare equal; NaN scores
// count as -inf): the result is exact.
// A row longer than one block holds in registers (1024 x 64 keys) is taken
// in pieces in key order, carrying the top_k kept so far into the next
// piece (topk_row_long).
//
// The kernel is bound by vector-ALU issue (a 64-lane instruction occupies a
// 16-lane SIMD for four cycles), so each pass over the keys is kept to a few
// instructions per key.
#include "dsa_kernels.h"

#include <type_traits>

namespace dsa {
namespace {

constexpr int kBins = 256;
constexpr int kMaxLevels = 4;

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

// ---- wave primitives on DPP (every lane of the wave active) ----

// (kDpp* controls, dpp_perm on ints and group_sum are in dsa_kernels.h.
// The float form has a name of its own: a dpp_perm declared in this
// namespace would hide the int one, and its call would become a recursion.)
template <int CTRL>
__device__ inline float dpp_perm_f(float x) {
    return __builtin_bit_cast(float, dsa::dpp_perm<CTRL>(__builtin_bit_cast(int, x)));
}
__device__ inline float readlane_f(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

struct MinOp { __device__ float operator()(float a, float b) const { return fminf(a, b); } };
struct MaxOp { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// op over the wave, wave-uniform: every lane of a row gets the row's result
// through four in-row exchanges, then the four rows are read out.
template <typename Op>
__device__ inline float wave_reduce(float x, Op op) {
    x = op(x, dpp_perm_f<kDppXor1>(x));
    x = op(x, dpp_perm_f<kDppXor2>(x));
    x = op(x, dpp_perm_f<kDppHalfMirror>(x));
    x = op(x, dpp_perm_f<kDppMirror>(x));
    return op(op(readlane_f(x, 0), readlane_f(x, 16)), op(readlane_f(x, 32), readlane_f(x, 48)));
}


// Inclusive sum over the lanes at or below this one: row shifts inside each
// 16-lane row (zeros shifted in), then the totals of earlier rows broadcast.
__device__ inline int wave_inclusive_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

template <int NT, int EPT>
struct TopkSmem {
    static constexpr int NW = NT / 64;
    static constexpr int NE = NT * EPT;                           // elements of a row
    static constexpr int NB = NE / 32;                            // bitmap words, bit k is element k
    static constexpr int kSlice = NT < 64 * EPT ? NT : 64 * EPT;  // a wave's most boundary-bin keys
    static_assert(NE <= 65536, "element indices are stored in 16 bits");
    float red[2][2][NW] __attribute__((aligned(16)));   // min / max partials, double buffered
    int cnt[2][NW];                                     // bisection counts, double buffered
    int wsum[NW];                                       // block-scan partials
    int hist[kBins] __attribute__((aligned(16)));
    float cand[NT + 64] __attribute__((aligned(16)));   // the boundary bin's values, NaN past them
    int candk[NT] __attribute__((aligned(16)));         // and their elements
    uint32_t keep[NB];                                  // kept elements
    uint32_t tie[NB];                                   // elements equal to T, where only some stay
    union {
        struct {                                        // gathering the boundary bin
            float slice[NW][kSlice];                    // each wave's boundary-bin values
            uint16_t slicek[NW][kSlice];                // and elements
            int wcnt[NW];                               // and their number
        } g;
        struct {                                        // writing the selection
            int outk[kMaxTopK];                         // kept keys in output order
        } c;
    } u;
    int bstar, above, inbin;                            // the level's boundary bin
    int ties;                                           // the ties at T kept, when only some are
};

// Compare predicates of the lane-mask builtins (LLVM's numbering).
constexpr int kCmpOge = 3;   // float, ordered >=

// Lanes l and l + 1 of x take the low and high halves of the wave-uniform
// mask m (v_writelane).  The mask usually comes straight from a compare;
// the compiler does not see the lane writes inside the asm, so the asm
// itself leaves the wait states a VALU-written SGPR needs before a lane
// access reads it.
__device__ __forceinline__ void write_mask(uint32_t& x, uint64_t m, int l) {
    asm("s_nop 4\n\tv_writelane_b32 %0, %1, %3\n\tv_writelane_b32 %0, %2, %4"
        : "+v"(x)
        : "s"((uint32_t)m), "s"((uint32_t)(m >> 32)), "i"(l), "i"(l + 1));
}

// Block-wide minimum and maximum (every thread gets both).
template <typename Sm>
__device__ inline void block_minmax(float& lo, float& hi, int& par, Sm& sm) {
    constexpr int NW = Sm::NW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    lo = wave_reduce(lo, MinOp{});
    hi = wave_reduce(hi, MaxOp{});
    if (lane == 0) { sm.red[par][0][wave] = lo; sm.red[par][1][wave] = hi; }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < NW; ++v) { lo = fminf(lo, sm.red[par][0][v]); hi = fmaxf(hi, sm.red[par][1][v]); }
    lo = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, lo)));
    hi = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, hi)));
    par ^= 1;
}

// The bin of a live value: trunc(v * scale + off) clamped to [0, 255], with
// off = -lo * scale, in one fused multiply-add.  A non-decreasing function of
// v (each rounding is monotone), so higher bins hold larger values and equal
// values share a bin.
__device__ inline int value_bin(float v, float scale, float off) {
    const int b = (int)__builtin_fmaf(v, scale, off);
    return min(max(b, 0), kBins - 1);
}

// The first float f of [a, b] at which fma(f, scale, off) >= n (a predicate
// that only grows with f), or b itself when no earlier float reaches n;
// every lane of the wave gets it.  A search over the order-preserving keys
// that tests 64 keys per round: the first round a window of 64 consecutive
// floats at the estimate (n - off) / scale, which usually brackets the
// answer, then 64 evenly spaced keys, each round keeping the stretch that
// ends at the first key that passes.  A span of 2^32 keys takes six rounds.
__device__ inline float first_reaching(float n, float a, float b, float scale, float off) {
    const int lane = threadIdx.x & 63;
    const uint32_t kend = order_key(b);
    uint32_t ka = order_key(a), kb = kend;
    const uint32_t kg = order_key(fminf(fmaxf((n - off) / scale, a), b));
    for (int round = 0; round < 16 && ka != kb; ++round) {
        uint32_t t;
        if (round == 0) {
            // kg - 32 + lane within [ka, kb] (unsigned compares throughout)
            const uint32_t w0 = kg >= ka + 32u ? kg - 32u : ka;
            t = w0 + (uint32_t)lane;
            t = t < kb ? t : kb;
        } else {
            t = ka + (uint32_t)(((uint64_t)(kb - ka) * (uint32_t)(lane + 1)) >> 6);   // lane 63 tests kb
        }
        const bool pass = t == kend || __builtin_fmaf(key_value(t), scale, off) >= n;
        const uint64_t m = __ballot(pass);
        if (m == 0) {   // only in the window round: everything up to its last key fails
            ka = (uint32_t)__builtin_amdgcn_readlane((int)t, 63) + 1u;
            continue;
        }
        const int j = __builtin_ctzll(m);
        const uint32_t tj = (uint32_t)__builtin_amdgcn_readlane((int)t, j);
        const uint32_t below = j > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)t, j - 1) + 1u : ka;
        ka = below;
        kb = tj;
    }
    return key_value(ka);
}

// Both edges of bin b at once: L, the first float of [lo, hiup] whose bin
// reaches b, and U, the first whose bin reaches b + 1 (lo for b = 0 and hiup
// for the last bin).  Lanes 0-31 test a window of 32 consecutive floats at
// L's estimate and lanes 32-63 one at U's; an edge whose window does not
// bracket it is searched in full (first_reaching).
__device__ inline void bin_edges(int b, float lo, float hiup, float scale, float off, float& L, float& U) {
    const int lane = threadIdx.x & 63, h = lane >> 5;
    const float n = (float)(b + h);
    const uint32_t ka = order_key(lo), kend = order_key(hiup);
    const uint32_t kg = order_key(fminf(fmaxf((n - off) / scale, lo), hiup));
    const uint32_t w0 = kg >= ka + 16u ? kg - 16u : ka;
    uint32_t t = w0 + (uint32_t)(lane & 31);
    t = t < kend ? t : kend;
    const bool pass = t == kend || __builtin_fmaf(key_value(t), scale, off) >= n;
    const uint64_t m = __ballot(pass);
    float e[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t mk = (uint32_t)(m >> (32 * k));
        const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)t, 32 * k);
        // bracketed: some key passes, and the first that does is the window's
        // first key only when that is lo itself
        if (mk != 0u && ((mk & 1u) == 0u || t0 == ka)) {
            e[k] = key_value((uint32_t)__builtin_amdgcn_readlane((int)t, 32 * k + __builtin_ctz(mk)));
        } else {
            e[k] = first_reaching((float)(b + k), lo, hiup, scale, off);
        }
    }
    L = b > 0 ? e[0] : lo;
    U = b < kBins - 1 ? e[1] : hiup;
}

// Element k of a row: its score and the key index written for it.
// Loads go through a buffer resource sized to the row's n elements, so a
// read past the row returns zero instead of touching memory beyond it.
__device__ inline __amdgpu_buffer_rsrc_t row_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
struct DirectRow {   // element k is key k0 + k
    const float* __restrict__ s;
    int k0;
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int n) const { return row_rsrc(s, 4 * n); }
    __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, int k) const {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 4 * k, 0, 0));   // raw bits
    }
    __device__ __forceinline__ int32_t key(int k) const { return k0 + k; }
};
// Where the kept keys go (global memory, or LDS through a generic pointer).
struct KeySink {
    int32_t* __restrict__ out;
    __device__ __forceinline__ void write(int t, int32_t key) const { out[t] = key; }
};
// A piece of a long row: element k < C is the kept key carry[k] (carried
// from earlier pieces, ascending), element C + j is key k0 + j.  Every
// carried key is below k0, so element order is key order.
struct CarryRow {
    const float* __restrict__ s;   // the whole row
    const int32_t* carry;          // LDS
    int C, k0;
    __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(int n) const { return row_rsrc(s, 4 * (k0 + n - C)); }
    __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t r, int k) const {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 4 * key(k), 0, 0));
    }
    // C <= kMaxTopK: the first test lets the compiler drop the select for
    // elements past kMaxTopK; the clamp keeps a discarded read in the array
    __device__ __forceinline__ int32_t key(int k) const {
        return (k < kMaxTopK && k < C) ? carry[min(k, kMaxTopK - 1)] : k0 + k - C;
    }
};
// Kept keys through a generic pointer: the LDS carry of a long row (which
// the next piece's row reads: no restrict) or the output.
struct LdsSink {
    int32_t* out;
    __device__ __forceinline__ void write(int t, int32_t key) const { out[t] = key; }
};

template <int NT, int EPT, typename Row, typename Sink, typename Sm>
__device__ __forceinline__ void topk_row(const Row& row, int n, int top_k, const Sink& sink, int32_t* count,
                                         Sm& sm) {
    static_assert(NT >= kBins && NT % 64 == 0 && EPT >= 1 && EPT <= 64, "topk geometry");
    static_assert(kBins == 4 * 64, "one wave scans the histogram, four bins per lane");
    static_assert((NT * EPT) % 64 == 0, "whole groups");
    constexpr int NW = NT / 64;
    static_assert(NW % 4 == 0 || NW < 4, "group counts are read four at a time");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float kNone = __int_as_float(0x7FC00000);
    if (n <= top_k) {   // every earlier key; the scores are not read
        for (int t = tid; t < top_k; t += NT) sink.write(t, t < n ? row.key(t) : -1);
        if (tid == 0 && count) *count = n;
        return;
    }
    // Scores in registers.  A NaN score ranks as -inf; keys past the row are
    // NaN, which every comparison below treats as "not a candidate".
    float f[EPT];
    {
        const auto rs = row.rsrc(n);
#pragma unroll
        for (int e = 0; e < EPT; ++e)   // no waits between the loads
            f[e] = row.load(rs, e * NT + tid);
    }
    // fmaxf against -inf turns NaN into -inf and leaves the rest
    const int lim = n - tid;   // element e is in the row when e * NT < lim
#pragma unroll
    for (int e = 0; e < EPT; ++e) f[e] = e * NT < lim ? fmaxf(f[e], -INFINITY) : kNone;
    if (tid < kBins) sm.hist[tid] = 0;

    // the live set is every key with lo <= value <= hi; krem of them are kept
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPT; ++e) { lo = fminf(lo, f[e]); hi = fmaxf(hi, f[e]); }
    int par = 0;
    block_minmax(lo, hi, par, sm);
    int krem = top_k;
    bool found = false, direct = false;
    float T = 0.f;

    for (int lev = 0; lev < kMaxLevels; ++lev) {
        if (!(lo < hi)) { T = lo; found = true; break; }   // every live value equal (-0 == +0)
        const float scale = (float)kBins / (hi - lo);
        const float off = -lo * scale;
        // finite positive scale and finite offset only (excludes infinities
        // and overflowing ranges)
        if (!(scale > 0.f && scale < 3.0e38f && fabsf(off) < 3.0e38f)) break;
        // Every value lies in the first level's range: there a key is live
        // unless it is padding (NaN).
        if (lev == 0) {
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (f[e] == f[e]) atomicAdd(&sm.hist[value_bin(f[e], scale, off)], 1);
        } else {
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (f[e] >= lo && f[e] <= hi) atomicAdd(&sm.hist[value_bin(f[e], scale, off)], 1);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds bins b0 .. b0+3 with b0 = 252 - 4l: lower lanes
            // hold higher bins, so an inclusive lane sum counts from the top
            const int b0 = kBins - 4 - 4 * lane;
            const int4 hv = *reinterpret_cast<const int4*>(&sm.hist[b0]);
            const int h[4] = {hv.x, hv.y, hv.z, hv.w};
            const int tot = h[0] + h[1] + h[2] + h[3];
            int gt = wave_inclusive_sum(tot) - tot;   // live keys in bins above b0 + 3
#pragma unroll
            for (int k = 3; k >= 0; --k) {
                if (gt < krem && gt + h[k] >= krem) { sm.bstar = b0 + k; sm.above = gt; sm.inbin = h[k]; }
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
            // Direct ranking.  One pass over the keys writes the bitmap of
            // the keys above the bin (a 64-lane mask per element group, kept
            // in lanes 2e and 2e+1 of mw until one store per lane) and
            // gathers the bin's keys with their elements: each wave into its
            // own slice of LDS with a running count, no atomics.  The slices
            // are packed into one list and each key of the bin is ranked
            // against the others: a key kept together with all its ties sets
            // its bit; when only some of the keys equal to T fit, those set
            // tie bits instead (the walk keeps the lowest).
            constexpr int NMW = (EPT + 31) / 32;
            uint32_t mw[NMW];
#pragma unroll
            for (int i = 0; i < NMW; ++i) mw[i] = 0u;
            // Bin membership as two compares per key.  Uf and L are the
            // first floats (at or above lo) whose bin reaches bstar + 1 and
            // bstar, found exactly by searching the fused multiply-add, and
            // Uf is capped just above hi: a key is above the bin when
            // f >= Uf and in it when L <= f < Uf.  Keys below lo fail both,
            // keys above hi (kept at an earlier level) pass the first, and
            // NaN padding fails both.
            const float hiup = key_value(order_key(hi) + 1u);
            float L, Uf;
            bin_edges(bstar, lo, hiup, scale, off, L, Uf);
            int wc = 0;
            int me = tid;
            asm volatile("" : "+v"(me));   // elements computed where stored, not kept per element
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const uint64_t up = __builtin_amdgcn_fcmpf(f[e], Uf, kCmpOge);
                write_mask(mw[e / 32], up, 2 * (e % 32));
                const uint64_t m = __builtin_amdgcn_fcmpf(f[e], L, kCmpOge) & ~up;
                if (m) {
                    if ((m >> lane) & 1) {
                        const int p = wc + count_below(m);
                        sm.u.g.slice[wave][p] = f[e];
                        sm.u.g.slicek[wave][p] = (uint16_t)(e * NT + me);
                    }
                    wc += (int)__popcll(m);
                }
            }
#pragma unroll
            for (int i = 0; i < NMW; ++i) {
                const int e = 32 * i + (lane >> 1);
                if (e < EPT) {
                    sm.keep[(e * NT + 64 * wave) / 32 + (lane & 1)] = mw[i];
                    sm.tie[(e * NT + 64 * wave) / 32 + (lane & 1)] = 0u;
                }
            }
            if (lane == 0) sm.u.g.wcnt[wave] = wc;
            if (tid == 0) sm.ties = 0;
            __syncthreads();
            if (tid < inbin) {
                // key tid sits in the first slice whose running total exceeds it
                int w = 0, base = 0, cum = 0;
#pragma unroll
                for (int v = 0; v < NW; ++v) {
                    cum += sm.u.g.wcnt[v];
                    const bool past = tid >= cum;
                    w = past ? v + 1 : w;
                    base = past ? cum : base;
                }
                sm.cand[tid] = sm.u.g.slice[w][tid - base];
                sm.candk[tid] = sm.u.g.slicek[w][tid - base];
            }
            if (tid < 64) sm.cand[inbin + tid] = kNone;   // whole groups of four past the bin
            __syncthreads();
            // each key of the bin is ranked by P lanes (a power of two, up to
            // 16), which split the comparisons four values at a time and
            // combine their counts in-row
            int lg = 0;
            while (lg < 4 && (inbin << (lg + 1)) <= NT) ++lg;
            const int P = 1 << lg;
            const int c = tid >> lg, part = tid & (P - 1);
            int gt = 0, ge = 0;
            const float v = sm.cand[min(c, max(inbin - 1, 0))];
            if (c < inbin) {
#pragma unroll 2
                for (int i = 4 * part; i < inbin; i += 4 * P) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.cand[i]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        gt += x[j] > v;
                        ge += x[j] >= v;
                    }
                }
            }
            gt = group_sum(gt, P);
            ge = group_sum(ge, P);
            // kept when every key at or above its score fits; when only some
            // of its ties fit (gt < krem < ge: its score is T), it is marked
            // as a tie, and the lowest krem - gt of them stay
            if (c < inbin && part == 0 && gt < krem) {
                const int k = sm.candk[c];
                if (ge <= krem) {
                    atomicOr(&sm.keep[k >> 5], 1u << (k & 31));
                } else {
                    atomicOr(&sm.tie[k >> 5], 1u << (k & 31));
                    sm.ties = krem - gt;   // the same for every tie
                }
            }
            __syncthreads();
            krem = __builtin_amdgcn_readfirstlane(sm.ties);
            direct = true;
            break;
        }
        // narrow the live range to the bin's values
        float nlo = INFINITY, nhi = -INFINITY;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const bool a = f[e] >= lo && f[e] <= hi && value_bin(f[e], scale, off) == bstar;
            nlo = a ? fminf(nlo, f[e]) : nlo;
            nhi = a ? fmaxf(nhi, f[e]) : nhi;
        }
        if (tid < kBins) sm.hist[tid] = 0;
        lo = nlo;
        hi = nhi;
        block_minmax(lo, hi, par, sm);
    }

    // Without direct ranking (a bin of equal values, the bisection), keep
    // every key > T and the first krem keys == T in key order (NaN padding
    // is neither): lane 0 of each wave stores its group's 64-lane masks,
    // bits e*NT + 64w .. +63 of the kept and tie bitmaps.
    constexpr int NB = Sm::NB;
    int keep = krem;   // the ties kept
    if (!direct) {
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
        keep = krem;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            asm volatile("" : "+v"(f[e]));   // one element at a time: no hoisted masks
            const uint64_t m = __ballot(f[e] > T);
            const uint64_t q = __ballot(f[e] == T);
            if (lane == 0) {
                const int w = (e * NT + 64 * wave) / 32;
                sm.keep[w] = (uint32_t)m;
                sm.keep[w + 1] = (uint32_t)(m >> 32);
                sm.tie[w] = (uint32_t)q;
                sm.tie[w + 1] = (uint32_t)(q >> 32);
            }
        }
        __syncthreads();
    }

    // The walk: thread t owns bitmap words t*WPT .. t*WPT+WPT-1 (consecutive
    // keys).  One block scan of its (kept, tie) counts, packed as
    // kept + (tie << kEqShift), places its keys; the ties it keeps are the
    // first (keep - ties before it) of its own.  Sums never carry between
    // the fields: fewer than top_k <= 2048 keys are kept from the first map.
    constexpr int kEqShift = 13;
    static_assert(kMaxTopK < (1 << kEqShift) && (int64_t)Sm::NE << kEqShift <= 0x7FFFFFFF, "count packing");
    constexpr int WPT = (NB + NT - 1) / NT;
    const uint32_t* kwords = sm.keep;
    const uint32_t* twords = sm.tie;
    const bool ties = !direct || keep > 0;
    uint32_t kw[WPT], tw[WPT];
    int ck = 0, ct = 0;
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        const int w = tid * WPT + j;
        kw[j] = w < NB ? kwords[w] : 0u;
        tw[j] = (ties && w < NB) ? twords[w] : 0u;
        ck += __popc(kw[j]);
        ct += __popc(tw[j]);
    }
    const int mine = ck + (ct << kEqShift);
    const int incl = wave_inclusive_sum(mine);
    if (lane == 63) sm.wsum[wave] = incl;
    __syncthreads();
    int before = incl - mine;
#pragma unroll
    for (int v = 0; v < NW; ++v) before += v < wave ? sm.wsum[v] : 0;
    const int pk = before & ((1 << kEqShift) - 1), pt = before >> kEqShift;
    int q = min(max(keep - pt, 0), ct);    // ties this thread keeps
    int pos = pk + min(pt, keep);          // kept keys before its words
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
        uint32_t m = kw[j];
        if (ties) {
            uint32_t t = tw[j];
            const int c = __popc(t);
            if (c <= q) {
                m |= t;
                q -= c;
            } else {
                for (; q > 0; --q) { m |= t & (0u - t); t &= t - 1; }   // the lowest q of them
            }
        }
        const int k0w = (tid * WPT + j) * 32;
        while (m) {
            const int k = k0w + __builtin_ctz(m);
            m &= m - 1;
            sm.u.c.outk[pos++] = row.key(k);
        }
    }
    // the top_k kept keys leave in one coalesced pass
    __syncthreads();
    for (int t = tid; t < top_k; t += NT) sink.write(t, sm.u.c.outk[t]);
    if (tid == 0 && count) *count = top_k;
}

// Six waves per SIMD (three 512-thread or six 256-thread blocks per CU) need
// at most 80 VGPRs.
template <int NT, int EPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT <= 512 && EPT == 32 ? 6 : 4, 8))) void topk_prefill_kernel(
    TopkArgs a) {
    __shared__ TopkSmem<NT, EPT> sm;
    const int r = blockIdx.x;
    const int64_t p = a.pos0 + r;
    const int n = (int)(p + 1);
    const float* srow = (n > a.top_k) ? a.S + (int64_t)(r - a.s_row0) * a.ldS : nullptr;
    topk_row<NT, EPT>(DirectRow{srow, 0}, n, a.top_k, KeySink{a.idx + (int64_t)r * a.top_k},
                      a.count ? a.count + r : nullptr, sm);
}

// A row of n keys, of any length up to kMaxSelectKeys, in pieces in key
// order: the first NE = NT * EPT keys, then each time the top_k keys kept so
// far followed by the next NE - top_k keys (a row of at most NE keys is one
// piece).  The top_k of the kept keys and a piece are the top_k of every key
// read so far (a key left out already has top_k better ones), and the
// carried keys are lower than the piece's and come first in element order,
// so a tie still goes to the lower key.  One topk_row instance serves every
// piece: its sink is the carry array for all but the last.
// carry: kMaxTopK ints of LDS.
// (A separate function per piece: inlined into the loop, the compiler hoists
// the pass's per-element addresses out of it and spills.)
template <int NT, int EPT, typename Sm>
__device__ __noinline__ void topk_piece(const float* s, int32_t* carry, int C, int k0, int n, int top_k,
                                        int32_t* out, int32_t* count, Sm& sm) {
    topk_row<NT, EPT>(CarryRow{s, carry, C, k0}, n, top_k, LdsSink{out}, count, sm);
}
template <int NT, int EPT, typename Sm>
__device__ __forceinline__ void topk_row_long(const float* s, int n, int top_k, int32_t* out, int32_t* count,
                                              Sm& sm, int32_t* carry) {
    constexpr int NE = NT * EPT;
    static_assert(NE > kMaxTopK, "a piece must hold more than the carried keys");
    for (int k0 = 0, C = 0;;) {   // each pass reads at least NE - top_k new keys
        const int piece = min(n - k0, NE - C);
        const bool last = k0 + piece >= n;
        topk_piece<NT, EPT>(s, carry, C, k0, C + piece, top_k, last ? out : carry, last ? count : nullptr, sm);
        if (last) return;
        k0 += piece;
        C = top_k;
        __syncthreads();   // the carried keys are written
    }
}

// Rows longer than the largest single-block shape (1024 x 64 keys).
__global__ __launch_bounds__(1024) void topk_long_kernel(TopkArgs a) {
    __shared__ TopkSmem<1024, 64> sm;
    __shared__ int32_t carry[kMaxTopK];
    const int r = blockIdx.x;
    const int64_t p = a.pos0 + r;
    const int n = (int)(p + 1);
    const float* srow = (n > a.top_k) ? a.S + (int64_t)(r - a.s_row0) * a.ldS : nullptr;
    topk_row_long<1024, 64>(srow, n, a.top_k, a.idx + (int64_t)r * a.top_k, a.count ? a.count + r : nullptr, sm,
                            carry);
}

// ---- Decode: one selection per sequence, spread over segment blocks ----
//
// A sequence with more than top_k keys is split into segments of kDecSeg
// keys, one block each.  Every segment of a sequence bins its keys on one shared
// value-linear map: kDecBins bins between the minimum and maximum of a fixed
// sample of the sequence's scores.  Keys outside that range fall into the
// end bins, so the map stays monotone and every key is counted, and the
// segments' histograms add up to the sequence's.  Two launches:
//   A. each segment block stores its histogram;
//   B. each segment block sums its sequence's histograms and finds the bin
//      holding the top_k-th key; its keys above that bin go to the
//      sequence's list of sure keys and its keys in that bin (with scores)
//      to the candidate list, at offsets the histograms give, so both lists
//      are in key order.
// The decode attention blocks finish the selection: each ranks the
// candidates (score, then lower key), keeps as many as the count still
// allows, and merges them into the sure keys by binary search, keeping the
// slots of its own chunk.  A sequence whose sample gives no usable range, or
// whose boundary bin holds more than kDecCap keys, is selected in launch B
// by its first segment block over all of its keys instead (slower, same
// result), straight into idx and count.
constexpr int kDecSeg = 8192;                 // keys per segment block
constexpr int kDecT = 512;                    // threads of a segment block (one sample key each)
constexpr int kDecEPT = kDecSeg / kDecT;
constexpr int kDecBins = 1024;                // bins of the shared map
static_assert(kDecBins == 16 * 64 && kDecBins == 2 * kDecT, "one wave scans the bins, sixteen per lane");
static_assert(kDecSeg / 32 <= kDecT, "decode block shape");

// The shared bin of a (NaN-free) score: clamped in float, so +-inf and
// values outside the sample range land in the end bins.
__device__ inline int dec_bin(float v, float scale, float off) {
    return (int)fminf(fmaxf(__builtin_fmaf(v, scale, off), 0.f), (float)(kDecBins - 1));
}

// The sample range of sequence b, identical in every block: the minimum and
// maximum of kDecT evenly spaced scores (NaN ignored).
__device__ inline void dec_sample_range(const float* srow, int ctx, float& lo, float& hi, float (&red)[2][kDecT / 64]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float v = srow[(int)((int64_t)tid * ctx / kDecT)];
    lo = wave_reduce(v == v ? v : INFINITY, MinOp{});
    hi = wave_reduce(v == v ? v : -INFINITY, MaxOp{});
    if (lane == 0) { red[0][wave] = lo; red[1][wave] = hi; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kDecT / 64; ++w) { lo = fminf(lo, red[0][w]); hi = fmaxf(hi, red[1][w]); }
}

// Pass A: block -> (sequence b, segment g).
__global__ __launch_bounds__(kDecT) __attribute__((amdgpu_waves_per_eu(2, 8))) void topk_dec_hist_kernel(
        const float* S, SeqMeta m, DecWork w) {
    __shared__ int hist[kDecBins];
    __shared__ float red[2][kDecT / 64];
    const int tid = threadIdx.x;
    const int b = seq_of_block(m, blockIdx.x), g = blockIdx.x - m.blk0[b];
    const int ctx = m.ctx[b];
    const float* srow = S + m.s_off[b];
    const int k0 = g * kDecSeg, n = min(ctx - k0, kDecSeg);
    float f[kDecEPT];
    {
        const auto rs = row_rsrc(srow + k0, 4 * n);   // reads past the segment return 0
#pragma unroll
        for (int e = 0; e < kDecEPT; ++e)
            f[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (e * kDecT + tid), 0, 0));
    }
    for (int i = tid; i < kDecBins; i += kDecT) hist[i] = 0;
    float lo, hi;
    dec_sample_range(srow, ctx, lo, hi, red);   // ends with a barrier
    const float scale = (float)kDecBins / (hi - lo), off = -lo * scale;
    const bool degenerate = !(lo < hi) || !(scale > 0.f && scale < 3.0e38f && fabsf(off) < 3.0e38f);
    if (!degenerate) {
#pragma unroll
        for (int e = 0; e < kDecEPT; ++e)
            if (e * kDecT + tid < n) atomicAdd(&hist[dec_bin(fmaxf(f[e], -INFINITY), scale, off)], 1);
    }
    __syncthreads();
    for (int i = tid; i < kDecBins; i += kDecT) w.hist[(int64_t)blockIdx.x * kDecBins + i] = hist[i];
    if (g == 0 && tid == 0) w.info[b] = DecSeqInfo{scale, off, degenerate ? 1 : 0, 0, 0, 0, {0, 0}};
}

// Pass B: block -> (sequence b, segment g), for sequences of two or more.
__global__ __launch_bounds__(kDecT) __attribute__((amdgpu_waves_per_eu(2, 8))) void topk_dec_split_kernel(
        const float* S, SeqMeta m, int top_k, DecWork w, int32_t* idx, int32_t* count) {
    __shared__ int htot[kDecBins] __attribute__((aligned(16)));
    __shared__ int hbef[kDecBins] __attribute__((aligned(16)));
    __shared__ uint64_t bm_sure[kDecSeg / 64], bm_cand[kDecSeg / 64];
    __shared__ float cval[kDecSeg];
    __shared__ int wsum[kDecT / 64];
    __shared__ int s_bstar, s_above, s_inbin, s_bef_above, s_bef_in;
    __shared__ TopkSmem<kDecT, 32> fsm;   // the fallback selection
    __shared__ int32_t carry[kMaxTopK];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = seq_of_block(m, blockIdx.x), g = blockIdx.x - m.blk0[b];
    const int ctx = m.ctx[b], G = m.blk0[b + 1] - m.blk0[b];
    const DecSeqInfo info = w.info[b];
    // the whole sequence by its first segment block, straight into idx/count
    auto fallback = [&]() {
        if (g == 0)
            topk_row_long<kDecT, 32>(S + m.s_off[b], ctx, top_k, idx + (int64_t)b * top_k, count + b, fsm, carry);
    };
    if (info.degenerate) {
        fallback();
        return;
    }
    const int k0 = g * kDecSeg, n = min(ctx - k0, kDecSeg);
    float f[kDecEPT];
    {
        const auto rs = row_rsrc(S + m.s_off[b] + k0, 4 * n);
#pragma unroll
        for (int e = 0; e < kDecEPT; ++e)
            f[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (e * kDecT + tid), 0, 0));
    }
    if (tid == 0) s_inbin = kDecCap + 1;   // stays so (fallback) if no bin were found
    // the sequence's histogram, and the part of it from earlier segments
    const int* h0 = w.hist + (int64_t)m.blk0[b] * kDecBins;
#pragma unroll
    for (int r = 0; r < kDecBins / kDecT; ++r) {
        const int i = r * kDecT + tid;
        int tot = 0, bef = 0;
        for (int s0 = 0; s0 < G; s0 += 8) {   // eight segments' counts, loads issued together
            int h[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) h[s] = s0 + s < G ? h0[(int64_t)(s0 + s) * kDecBins + i] : 0;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                tot += h[s];
                bef += s0 + s < g ? h[s] : 0;
            }
        }
        htot[i] = tot;
        hbef[i] = bef;
    }
    __syncthreads();
    if (wave == 0) {
        // lane l holds bins b0 .. b0+15 with b0 = kDecBins - 16(l+1): an
        // inclusive lane sum counts from the top
        const int b0 = kDecBins - 16 * (lane + 1);
        int h[16], hb[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int4 x = *reinterpret_cast<const int4*>(&htot[b0 + 4 * q]);
            const int4 y = *reinterpret_cast<const int4*>(&hbef[b0 + 4 * q]);
            h[4 * q] = x.x; h[4 * q + 1] = x.y; h[4 * q + 2] = x.z; h[4 * q + 3] = x.w;
            hb[4 * q] = y.x; hb[4 * q + 1] = y.y; hb[4 * q + 2] = y.z; hb[4 * q + 3] = y.w;
        }
        int t16 = 0, b16 = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) { t16 += h[k]; b16 += hb[k]; }
        int gt = wave_inclusive_sum(t16) - t16, bgt = wave_inclusive_sum(b16) - b16;
#pragma unroll
        for (int k = 15; k >= 0; --k) {
            if (gt < top_k && gt + h[k] >= top_k) {
                s_bstar = b0 + k; s_above = gt; s_inbin = h[k]; s_bef_above = bgt; s_bef_in = hb[k];
            }
            gt += h[k];
            bgt += hb[k];
        }
    }
    __syncthreads();
    const int bstar = __builtin_amdgcn_readfirstlane(s_bstar);
    const int above = __builtin_amdgcn_readfirstlane(s_above);
    const int inbin = __builtin_amdgcn_readfirstlane(s_inbin);
    const int bef_above = __builtin_amdgcn_readfirstlane(s_bef_above);
    const int bef_in = __builtin_amdgcn_readfirstlane(s_bef_in);
    if (inbin > kDecCap) {
        if (g == 0 && tid == 0) w.info[b].fallback = 1;
        fallback();
        return;
    }
    if (g == 0 && tid == 0) { w.info[b].above = above; w.info[b].inbin = inbin; }
    // this segment's sure keys and candidates as bitmaps (bit k: element k)
#pragma unroll
    for (int e = 0; e < kDecEPT; ++e) {
        asm volatile("" : "+v"(f[e]));   // one element at a time: no hoisted masks
        const bool in = e * kDecT + tid < n;
        const float v = fmaxf(f[e], -INFINITY);
        const int bin = dec_bin(v, info.scale, info.off);
        const bool sure = in && bin > bstar, cd = in && bin == bstar;
        const uint64_t ms = __ballot(sure), mc = __ballot(cd);
        if (lane == 0) {
            bm_sure[(e * kDecT + 64 * wave) / 64] = ms;
            bm_cand[(e * kDecT + 64 * wave) / 64] = mc;
        }
        if (cd) cval[e * kDecT + tid] = v;
    }
    __syncthreads();
    // thread t < kDecSeg / 32 owns bitmap word t (keys 32t .. 32t+31); one
    // block scan of its (sure, candidate) counts, packed as sure + (cand <<
    // 13): this segment holds fewer than top_k <= 2048 sure keys
    constexpr int kShift = 13;
    static_assert(kMaxTopK < (1 << kShift) && kDecCap < (1 << (31 - kShift)), "count packing");
    const uint32_t* ws = reinterpret_cast<const uint32_t*>(bm_sure);
    const uint32_t* wc = reinterpret_cast<const uint32_t*>(bm_cand);
    uint32_t xs = tid < kDecSeg / 32 ? ws[tid] : 0u, xc = tid < kDecSeg / 32 ? wc[tid] : 0u;
    const int mine = __popc(xs) + (__popc(xc) << kShift);
    const int incl = wave_inclusive_sum(mine);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = incl - mine;
#pragma unroll
    for (int v = 0; v < kDecT / 64; ++v) before += v < wave ? wsum[v] : 0;
    int ps = bef_above + (before & ((1 << kShift) - 1)), pc = bef_in + (before >> kShift);
    int32_t* sure = w.sure + (int64_t)b * top_k;
    DecCand* cand = w.cand + (int64_t)b * kDecCap;
    // (the counts match the histograms bin for bin, so every offset is in
    // range; the bounds below only guard the lists)
    while (xs) {
        const int k = 32 * tid + __builtin_ctz(xs);
        xs &= xs - 1;
        if (ps < above) sure[ps] = k0 + k;
        ++ps;
    }
    while (xc) {
        const int k = 32 * tid + __builtin_ctz(xc);
        xc &= xc - 1;
        if (pc < inbin) cand[pc] = DecCand{k0 + k, cval[k]};
        ++pc;
    }
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
    return hipErrorInvalidValue;   // longer rows: topk_long_kernel
}

}  // namespace

hipError_t launch_topk_prefill(const TopkArgs& a, int n_max, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    if (n_max > 65536) {
        if (n_max > kMaxSelectKeys) return hipErrorInvalidValue;
        hipLaunchKernelGGL(topk_long_kernel, dim3(a.rows), dim3(1024), 0, s, a);
        return hipGetLastError();
    }
    return dispatch_shape(n_max, [&](auto nt, auto ept) {
        constexpr int NT = decltype(nt)::value, EPT = decltype(ept)::value;
        hipLaunchKernelGGL((topk_prefill_kernel<NT, EPT>), dim3(a.rows), dim3(NT), 0, s, a);
        return hipGetLastError();
    });
}

int topk_decode_segments(int ctx, int top_k) { return ctx > top_k ? (ctx + kDecSeg - 1) / kDecSeg : 0; }

namespace {
constexpr size_t align256(size_t x) { return (x + 255) / 256 * 256; }
DecWork carve(void* base, int B, int blocks, int top_k) {
    char* p = static_cast<char*>(base);
    DecWork w;
    w.hist = reinterpret_cast<int*>(p);
    p += align256((size_t)blocks * kDecBins * sizeof(int));
    w.info = reinterpret_cast<DecSeqInfo*>(p);
    p += align256((size_t)B * sizeof(DecSeqInfo));
    w.sure = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * top_k * sizeof(int32_t));
    w.cand = reinterpret_cast<DecCand*>(p);
    return w;
}
}  // namespace

DecWork topk_decode_work(void* work, int B, int blocks, int top_k) { return carve(work, B, blocks, top_k); }

size_t topk_decode_work_bytes(int B, int blocks, int top_k) {
    return align256((size_t)blocks * kDecBins * sizeof(int)) + align256((size_t)B * sizeof(DecSeqInfo)) +
           align256((size_t)B * top_k * sizeof(int32_t)) + align256((size_t)B * kDecCap * sizeof(DecCand));
}

hipError_t launch_topk_decode(const float* S, const SeqMeta& m, int top_k, int32_t* idx, int32_t* count,
                              void* work, hipStream_t s) {
    if (m.B <= 0) return hipSuccess;
    const int blocks = m.blk0[m.B];
    const DecWork w = carve(work, m.B, blocks, top_k);
    if (blocks > 0) {
        hipLaunchKernelGGL(topk_dec_hist_kernel, dim3(blocks), dim3(kDecT), 0, s, S, m, w);
        hipLaunchKernelGGL(topk_dec_split_kernel, dim3(blocks), dim3(kDecT), 0, s, S, m, top_k, w, idx, count);
    }
    return hipGetLastError();
}

}  // namespace dsa
