// cache_write.hip - the upstream cache write of new tokens on gfx950.
//
// "GLM-5.2-Vision: llama.cpp vs vLLM line-by-line pipeline trace", section 4
// (KV compression path): the kv_a projection output of a token is split into
// kv_cmpr (the first Dl columns) and k_pe (the last Dr); k_pe and the query's
// q_pe are rotated by RoPE and kv_cmpr is RMS-normalised (with the kv_a norm
// weight) after the split.  Section 5 (RoPE convention): the rotation is the
// NORM flavour, adjacent pairs (x[2i], x[2i+1]), for the attention and for
// the indexer alike.  The pair-i angle at position p over a rope width d is
// p * theta^(-2i/d); theta, the norm epsilon and the indexer rope width are
// arguments (the pages do not print them).
//
// One 256-thread block per token.  The work is a few kilobytes of HBM traffic
// per token (the query's rope columns dominate), so the kernel is bound by
// HBM and every element is moved once, as 16-byte vectors:
//  - wave 0 normalises the latent part and writes it to cache row pos;
//  - wave 1 rotates k_pe into the same row and writes the indexer key row;
//  - all threads rotate the query's rope columns of every head and the
//    indexer query's leading columns, in place.
// The arithmetic (angles, sines and cosines, the rotation, the sum of squares
// and the scaling) runs in double precision and each result is rounded once
// to bf16 (nearest, ties to even): the rounding of a double result to 8
// significant bits then matches the exactly rounded value except when that
// value lies within about 1e-16 (relative) of a rounding midpoint.  The
// double work is a few dozen operations per element, far below the HBM time.
#include "dsa_kernels.h"

#include <math.h>

namespace dsa {
namespace {

constexpr int kCwThreads = 256;

__device__ inline double bf16_to_f64(uint32_t b) { return (double)__uint_as_float(b << 16); }

// double -> bf16 bits, round to nearest with ties to even on the 53-bit
// significand.  Zero and the normal bf16 range are exact; values below the
// normal range flush to a signed zero, values above it become infinities.
__device__ inline uint32_t f64_to_bf16(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const int e = (int)((u >> 52) & 0x7FF);
    if (e == 0) return sign;
    const uint64_t m = (u & 0xFFFFFFFFFFFFFull) | (1ull << 52);
    uint64_t keep = m >> 45;                                  // 8 significant bits
    const uint64_t rem = m & ((1ull << 45) - 1), half = 1ull << 44;
    if (rem > half || (rem == half && (keep & 1))) ++keep;
    int eb = e - 1023 + 127;
    if (keep == 256) { keep = 128; ++eb; }
    if (eb <= 0) return sign;
    if (eb >= 255) return sign | 0x7F80u;
    return sign | ((uint32_t)eb << 7) | (uint32_t)(keep & 127);
}

// Rotate the four adjacent pairs of one 16-byte vector (8 bf16); pair k
// uses table entry i0 + k.
__device__ inline u32x4 rope_vec(const u32x4 x, const double2* cs, int i0) {
    u32x4 y;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const double a = bf16_to_f64(x[k] & 0xFFFFu), b = bf16_to_f64(x[k] >> 16);
        const double c = cs[i0 + k].x, s = cs[i0 + k].y;
        y[k] = f64_to_bf16(a * c - b * s) | (f64_to_bf16(a * s + b * c) << 16);
    }
    return y;
}

template <int H, int DL, int DR, int HI, int DI>
__global__ __launch_bounds__(kCwThreads) void cache_write_kernel(CacheWriteArgs a) {
    static_assert(DL % 8 == 0 && DR % 8 == 0 && DI % 8 == 0, "16-byte vectors");
    static_assert(DL / 8 <= 64 && DR / 8 + DI / 8 <= 64, "one wave per part");
    constexpr int DQK = DL + DR;
    __shared__ double2 cs_r[DR / 2 > 0 ? DR / 2 : 1];    // (cos, sin) over the Dr-wide rope
    __shared__ double2 cs_i[DI / 2];                     // ... over the indexer rope width
    const int t = blockIdx.x;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int p = a.pos[t];
    const double pd = (double)p;
    const int dir = a.d_idx_rope;
    const double lth = log2((double)a.theta);
    if (w == 0 && l < DR / 2) {
        double s, c;
        sincos(pd * exp2(lth * (-2.0 * l / DR)), &s, &c);
        cs_r[l] = make_double2(c, s);
    } else if (w == 1 && l < dir / 2) {
        double s, c;
        sincos(pd * exp2(lth * (-2.0 * l / dir)), &s, &c);
        cs_i[l] = make_double2(c, s);
    }
    __syncthreads();
    const bool write_row = p >= 0 && p < a.N;
    if (write_row && w == 0) {
        // latent part: x / sqrt(mean(x^2) + eps) * weight
        const uint16_t* src = a.kv_a + (int64_t)t * DQK;
        u32x4 x = {0u, 0u, 0u, 0u};
        double ss = 0.0;
        if (l < DL / 8) {
            x = ldg16(src + 8 * l);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const double lo = bf16_to_f64(x[k] & 0xFFFFu), hi = bf16_to_f64(x[k] >> 16);
                ss += lo * lo + hi * hi;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        const double r = 1.0 / sqrt(ss / DL + (double)a.eps);
        if (l < DL / 8) {
            u32x4 y;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const double lo = bf16_to_f64(x[k] & 0xFFFFu) * r * (double)a.norm_w[8 * l + 2 * k];
                const double hi = bf16_to_f64(x[k] >> 16) * r * (double)a.norm_w[8 * l + 2 * k + 1];
                y[k] = f64_to_bf16(lo) | (f64_to_bf16(hi) << 16);
            }
            *reinterpret_cast<u32x4*>(a.kv + (int64_t)p * DQK + 8 * l) = y;
        }
    } else if (write_row && w == 1) {
        if (l < DR / 8) {            // k_pe -> rope -> cache row
            const u32x4 x = ldg16(a.kv_a + (int64_t)t * DQK + DL + 8 * l);
            *reinterpret_cast<u32x4*>(a.kv + (int64_t)p * DQK + DL + 8 * l) = rope_vec(x, cs_r, 4 * l);
        } else if (a.kI && l < DR / 8 + DI / 8) {   // indexer key: leading columns roped
            const int v = l - DR / 8;
            const u32x4 x = ldg16(a.kI_new + (int64_t)t * DI + 8 * v);
            *reinterpret_cast<u32x4*>(a.kI + (int64_t)p * DI + 8 * v) = (8 * v < dir) ? rope_vec(x, cs_i, 4 * v) : x;
        }
    }
    // the query's rope columns of every head, and the indexer query
    if (a.q) {
        constexpr int VR = DR / 8;
        uint16_t* qt = a.q + (int64_t)t * H * DQK + DL;
        for (int i = tid; i < H * VR; i += kCwThreads) {
            const int h = i / VR, v = i % VR;
            uint16_t* ptr = qt + (int64_t)h * DQK + 8 * v;
            *reinterpret_cast<u32x4*>(ptr) = rope_vec(ldg16(ptr), cs_r, 4 * v);
        }
    }
    if (a.qI && dir > 0) {
        const int VI = dir / 8;
        uint16_t* qt = a.qI + (int64_t)t * HI * DI;
        for (int i = tid; i < HI * VI; i += kCwThreads) {
            const int h = i / VI, v = i % VI;
            uint16_t* ptr = qt + (int64_t)h * DI + 8 * v;
            *reinterpret_cast<u32x4*>(ptr) = rope_vec(ldg16(ptr), cs_i, 4 * v);
        }
    }
}

}  // namespace

hipError_t launch_cache_write(int shape_id, const CacheWriteArgs& a, hipStream_t s) {
    if (a.T <= 0) return hipSuccess;
    const dim3 grid((unsigned)a.T), block(kCwThreads);
    if (shape_id == 0) hipLaunchKernelGGL((cache_write_kernel<64, 512, 64, 32, 128>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((cache_write_kernel<4, 64, 16, 4, 32>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace dsa
