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
// HBM and every element is moved once, as 16-byte vectors.  Every load of
// the token is issued first; while they are in flight waves 2 and 3 build
// the (cos, sin) tables and wave 0 normalises the latent part into cache row
// pos; after one barrier wave 1 rotates k_pe into the same row and writes
// the indexer key row, and all threads rotate the query's rope columns of
// every head and the indexer query's leading columns, in place.
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

// double -> bf16 bits, round to nearest with ties to even.  Rounding to
// float first (nearest-even) and then to bf16 gives the correctly rounded
// result except when the float lands exactly on a bf16 midpoint (its low 16
// bits are 0x8000) without the double being there: then the second rounding
// would see a false tie.  In that case the float is moved one ulp toward the
// double before the bf16 rounding.  Exact for results in the normal bf16
// range.
__device__ inline uint32_t f64_to_bf16(double v) {
    const float r = (float)v;
    uint32_t u = __float_as_uint(r);
    if ((u & 0xFFFFu) == 0x8000u) {
        const double back = (double)r;
        if (back != v) u = (fabs(back) > fabs(v)) ? u - 1u : u + 1u;
    }
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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
    constexpr int VR = DR / 8;                                              // vectors per rope row
    constexpr int QV = (H * VR + kCwThreads - 1) / kCwThreads;              // query vectors per thread
    constexpr int IV = (HI * (DI / 8) + kCwThreads - 1) / kCwThreads;       // indexer-query vectors (max)
    __shared__ double2 cs_r[DR / 2 > 0 ? DR / 2 : 1];    // (cos, sin) over the Dr-wide rope
    __shared__ double2 cs_i[DI / 2];                     // ... over the indexer rope width
    const int t = blockIdx.x;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int p = a.pos[t];
    const int dir = a.d_idx_rope, VI = dir / 8;
    const bool write_row = p >= 0 && p < a.N;

    // 1. every load of the token first, so that they are in flight while
    //    the rotation tables are built
    u32x4 qv[QV], iv[IV], rv = {0u, 0u, 0u, 0u};
    uint16_t* qrow = a.q ? a.q + (int64_t)t * H * DQK + DL : nullptr;
    uint16_t* irow = a.qI ? a.qI + (int64_t)t * HI * DI : nullptr;
    if (a.q) {
#pragma unroll
        for (int j = 0; j < QV; ++j) {
            const int i = tid + j * kCwThreads;
            if (i < H * VR) qv[j] = ldg16(qrow + (int64_t)(i / VR) * DQK + 8 * (i % VR));
        }
    }
    if (a.qI) {
#pragma unroll
        for (int j = 0; j < IV; ++j) {
            const int i = tid + j * kCwThreads;
            if (i < HI * VI) iv[j] = ldg16(irow + (int64_t)(i / VI) * DI + 8 * (i % VI));
        }
    }
    if (write_row) {
        if (w == 0 && l < DL / 8) rv = ldg16(a.kv_a + (int64_t)t * DQK + 8 * l);                 // kv_cmpr
        else if (w == 1 && l < VR) rv = ldg16(a.kv_a + (int64_t)t * DQK + DL + 8 * l);          // k_pe
        else if (w == 1 && a.kI && l < VR + DI / 8) rv = ldg16(a.kI_new + (int64_t)t * DI + 8 * (l - VR));
    }

    // 2. rotation tables in double: pair i turns by p * theta^(-2i/d)
    const double pd = (double)p, lth = log2((double)a.theta);
    if (w == 2 && l < DR / 2) {
        double sn, cn;
        sincos(pd * exp2(lth * (-2.0 * l / DR)), &sn, &cn);
        cs_r[l] = make_double2(cn, sn);
    } else if (w == 3 && l < dir / 2) {
        double sn, cn;
        sincos(pd * exp2(lth * (-2.0 * l / dir)), &sn, &cn);
        cs_i[l] = make_double2(cn, sn);
    }
    // 3. latent part: x / sqrt(mean(x^2) + eps) * weight (no table needed)
    if (write_row && w == 0) {
        double ss = 0.0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const double lo = bf16_to_f64(rv[k] & 0xFFFFu), hi = bf16_to_f64(rv[k] >> 16);
            ss += lo * lo + hi * hi;
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        const double r = 1.0 / sqrt(ss / DL + (double)a.eps);
        if (l < DL / 8) {
            u32x4 y;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const double lo = bf16_to_f64(rv[k] & 0xFFFFu) * r * (double)a.norm_w[8 * l + 2 * k];
                const double hi = bf16_to_f64(rv[k] >> 16) * r * (double)a.norm_w[8 * l + 2 * k + 1];
                y[k] = f64_to_bf16(lo) | (f64_to_bf16(hi) << 16);
            }
            *reinterpret_cast<u32x4*>(a.kv + (int64_t)p * DQK + 8 * l) = y;
        }
    }
    __syncthreads();

    // 4. rotations and stores
    if (write_row && w == 1) {
        if (l < VR) {                                   // k_pe -> cache row
            *reinterpret_cast<u32x4*>(a.kv + (int64_t)p * DQK + DL + 8 * l) = rope_vec(rv, cs_r, 4 * l);
        } else if (a.kI && l < VR + DI / 8) {           // indexer key: leading columns roped
            const int v = l - VR;
            *reinterpret_cast<u32x4*>(a.kI + (int64_t)p * DI + 8 * v) = (8 * v < dir) ? rope_vec(rv, cs_i, 4 * v) : rv;
        }
    }
    if (a.q) {
#pragma unroll
        for (int j = 0; j < QV; ++j) {
            const int i = tid + j * kCwThreads;
            if (i < H * VR)
                *reinterpret_cast<u32x4*>(qrow + (int64_t)(i / VR) * DQK + 8 * (i % VR)) =
                    rope_vec(qv[j], cs_r, 4 * (i % VR));
        }
    }
    if (a.qI) {
#pragma unroll
        for (int j = 0; j < IV; ++j) {
            const int i = tid + j * kCwThreads;
            if (i < HI * VI)
                *reinterpret_cast<u32x4*>(irow + (int64_t)(i / VI) * DI + 8 * (i % VI)) =
                    rope_vec(iv[j], cs_i, 4 * (i % VI));
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
