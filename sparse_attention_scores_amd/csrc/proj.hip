// proj.hip - the projections after the attention on gfx950: the per-head
// value up-projection and the output projection.
//
// "GLM-5.2-Vision: llama.cpp vs vLLM line-by-line pipeline trace", section 6
// (build_attn): the latent-space attention output is decompressed per head
// with wv_b (kqv = v_mla . kqv), flattened over the heads and multiplied by
// the output projection wo; the config line gives v_head_dim 256 and hidden
// size 6144.  Weights are stored [out, in] with the input dimension
// contiguous, so both products are C = A B^T with A and B contiguous along
// the reduction: the operand layout the MFMA wants.
//
// One kernel, two instances:
//  - up-projection: per head h (grid z), A = o[:, h, :] (float32, rounded to
//    bf16 as it is staged), B = wv[h] [256, 512], C = out_v[:, h, :] (bf16);
//  - output projection: A = out_v flattened [T, H*256] (bf16), B = wo
//    [6144, H*256], C = y [T, 6144] (float32).
// Block tile 256 x BN (BN = 256 for the up-projection, 192 for the output
// projection so that 6144 columns make 32 tiles) x 64 along the reduction;
// eight waves, each owning 64 rows x BN/2 columns as 2 x BN/64 tiles of
// v_mfma_f32_32x32x16_bf16 with accumulators in VGPRs.  The reduction
// streams through two LDS stages: the loads of stage s+1 are in flight
// (in VGPRs) while stage s is multiplied, then written to the other stage;
// one barrier per stage.  A tile row holds 64 bf16 (eight 16-byte chunks);
// chunk c of row r sits at c ^ ((r >> 1) & 7), which makes the fragment
// reads (32 rows, one chunk per half wave) conflict-free (measured: 182 B
// per clock per CU, against 40 unswizzled).
#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kGemmThreads = 512;
constexpr int kBM = 256, kBK = 64;
constexpr int kGroupN = 8;   // tile columns per group of the output projection's tile order

__device__ inline int gswz(int r) { return (r >> 1) & 7; }

__device__ inline uint32_t f32x2_to_bf16x2(float a, float b) {
    const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    const uint32_t ra = (ua + 0x7FFFu + ((ua >> 16) & 1u)) >> 16;
    const uint32_t rb = (ub + 0x7FFFu + ((ub >> 16) & 1u)) >> 16;
    return ra | (rb << 16);
}

template <bool A_F32, bool C_F32, int BN>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_nt_kernel(GemmArgs g) {
    constexpr int MT = 2;                          // 32-row MFMA tiles per wave
    constexpr int NT = BN / 64;                    // 32-column MFMA tiles per wave
    constexpr int A_PT = kBM * 8 / kGemmThreads;   // 16-byte chunks per thread per stage
    constexpr int B_PT = BN * 8 / kGemmThreads;
    static_assert(kBM * 8 % kGemmThreads == 0 && BN * 8 % kGemmThreads == 0, "even staging");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kBK];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int wm = w & 3, wn = w >> 2;
    const int64_t z = blockIdx.z;
    int m0, n0;
    if constexpr (A_F32) {
        m0 = blockIdx.x * kBM;
        n0 = blockIdx.y * BN;
    } else {
        // XCD-aware tile order.  Workgroups are dealt to the 8 XCDs in turn
        // (workgroup b runs on XCD b % 8), and each XCD has its own L2.  Tile
        // ids are numbered so that XCD k gets a contiguous run of them, and
        // the run covers a compact rectangle: groups of kGroupN tile columns,
        // column-fastest inside a group.  With 16 x 32 tiles each XCD then
        // reads an 8 x 8 block of tiles: half of A's rows and a quarter of
        // B's, instead of all of B.
        const int mt = (g.M + kBM - 1) / kBM, ntn = g.N / BN;
        const int per = ((mt * ntn) + 7) / 8;
        const int b = blockIdx.x;
        const int tile = (b & 7) * per + (b >> 3);
        if ((b >> 3) >= per || tile >= mt * ntn) return;
        const int gw = min(kGroupN, ntn);
        const int grp = tile / (mt * gw), in = tile % (mt * gw);
        const int width = min(gw, ntn - grp * gw);          // the last group may be narrower
        m0 = (in / width) * kBM;
        n0 = (grp * gw + in % width) * BN;
    }
    const uint16_t* Bz = g.B + z * g.b_batch;

    u32x4 ra[A_PT][A_F32 ? 2 : 1], rb[B_PT];
    auto load_stage = [&](int s) {
        const int k0 = s * kBK;
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
            const int idx = tid + i * kGemmThreads, row = idx >> 3, ch = idx & 7;
            const int64_t m = min(m0 + row, g.M - 1);   // rows past M repeat the last one (not stored)
            if constexpr (A_F32) {
                const float* p = static_cast<const float*>(g.A) + z * g.a_batch + m * g.lda + k0 + 8 * ch;
                ra[i][0] = ldg16(p);
                ra[i][1] = ldg16(p + 4);
            } else {
                ra[i][0] = ldg16(static_cast<const uint16_t*>(g.A) + z * g.a_batch + m * g.lda + k0 + 8 * ch);
            }
        }
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            const int idx = tid + i * kGemmThreads, row = idx >> 3, ch = idx & 7;
            rb[i] = ldg16(Bz + (int64_t)(n0 + row) * g.ldb + k0 + 8 * ch);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_PT; ++i) {
            const int idx = tid + i * kGemmThreads, row = idx >> 3, ch = idx & 7;
            u32x4 v;
            if constexpr (A_F32) {
                v[0] = f32x2_to_bf16x2(__uint_as_float(ra[i][0][0]), __uint_as_float(ra[i][0][1]));
                v[1] = f32x2_to_bf16x2(__uint_as_float(ra[i][0][2]), __uint_as_float(ra[i][0][3]));
                v[2] = f32x2_to_bf16x2(__uint_as_float(ra[i][1][0]), __uint_as_float(ra[i][1][1]));
                v[3] = f32x2_to_bf16x2(__uint_as_float(ra[i][1][2]), __uint_as_float(ra[i][1][3]));
            } else {
                v = ra[i][0];
            }
            *reinterpret_cast<u32x4*>(&As[buf][row * kBK + 8 * (ch ^ gswz(row))]) = v;
        }
#pragma unroll
        for (int i = 0; i < B_PT; ++i) {
            const int idx = tid + i * kGemmThreads, row = idx >> 3, ch = idx & 7;
            *reinterpret_cast<u32x4*>(&Bs[buf][row * kBK + 8 * (ch ^ gswz(row))]) = rb[i];
        }
    };

    f32x16 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};
    const int S = g.K / kBK;
    if constexpr (A_F32) {
        load_stage(0);
        store_stage(0);
    } else {
        constexpr int IA = kBM * 8 / 64, IB = BN * 8 / 64;
        const uint16_t* Az = static_cast<const uint16_t*>(g.A) + z * g.a_batch;
        for (int ins = w; ins < IA + IB; ins += 8) {
            if (ins < IA) {
                const int row = ins * 8 + (l >> 3), pc = l & 7;
                const int64_t m = min(m0 + row, g.M - 1);
                gather16_to_lds(Az, (uint32_t)((m * g.lda + 8 * (pc ^ gswz(row))) * 2), lds_addr(&As[0][ins * 512]));
            } else {
                const int bi = ins - IA, row = bi * 8 + (l >> 3), pc = l & 7;
                gather16_to_lds(Bz, (uint32_t)(((int64_t)(n0 + row) * g.ldb + 8 * (pc ^ gswz(row))) * 2),
                                lds_addr(&Bs[0][bi * 512]));
            }
        }
        wait_vmcnt<0>();
    }
    __syncthreads();
    auto read_frags = [&](int buf, int kk, u32x4 (&af)[MT], u32x4 (&bfr)[NT]) {
        const int ch = 2 * kk + (l >> 5);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int row = 64 * wm + 32 * i + (l & 31);
            af[i] = *reinterpret_cast<const u32x4*>(&As[buf][row * kBK + 8 * (ch ^ gswz(row))]);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int row = (BN / 2) * wn + 32 * j + (l & 31);
            bfr[j] = *reinterpret_cast<const u32x4*>(&Bs[buf][row * kBK + 8 * (ch ^ gswz(row))]);
        }
    };
    if constexpr (A_F32) {
        for (int s = 0; s < S; ++s) {
            const int buf = s & 1;
            if (s + 1 < S) load_stage(s + 1);
#pragma unroll
            for (int kk = 0; kk < kBK / 16; ++kk) {
                u32x4 af[MT], bfr[NT];
                read_frags(buf, kk, af, bfr);
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[i][j] = mfma32_bf16(af[i], bfr[j], acc[i][j]);
            }
            if (s + 1 < S) store_stage(buf ^ 1);
            __syncthreads();
        }
    } else {
        // bf16 operands go global -> LDS directly (global_load_lds_dwordx4,
        // 1 KB = 8 tile rows per instruction); the row swizzle is applied on
        // the source side (the lane that fills physical chunk pc of row r
        // loads logical chunk pc ^ ((r >> 1) & 7)).  The next stage's loads
        // are spread over the first two k-steps of the current one, so
        // issuing them never holds a wave for long and they have the last two
        // k-steps to land; a vmcnt(0) wait and one barrier close each stage.
        constexpr int IA = kBM * 8 / 64, IB = BN * 8 / 64;      // instructions per stage
        constexpr int IW = (IA + IB + 7) / 8;                    // per wave
        const uint16_t* Az = static_cast<const uint16_t*>(g.A) + z * g.a_batch;
        auto dma = [&](int s, int buf, int q) {   // q-th instruction of this wave
            const int ins = w + 8 * q;
            if (ins >= IA + IB) return;
            const int k0 = s * kBK;
            if (ins < IA) {
                const int row = ins * 8 + (l >> 3), pc = l & 7;
                const int64_t m = min(m0 + row, g.M - 1);
                const uint32_t voff = (uint32_t)((m * g.lda + k0 + 8 * (pc ^ gswz(row))) * 2);
                gather16_to_lds(Az, voff, lds_addr(&As[buf][ins * 512]));
            } else {
                const int bi = ins - IA, row = bi * 8 + (l >> 3), pc = l & 7;
                const uint32_t voff = (uint32_t)(((int64_t)(n0 + row) * g.ldb + k0 + 8 * (pc ^ gswz(row))) * 2);
                gather16_to_lds(Bz, voff, lds_addr(&Bs[buf][bi * 512]));
            }
        };
        for (int s = 0; s < S; ++s) {
            const int buf = s & 1;
            // fragments of k-step kk+1 are read before the MFMAs of kk
            u32x4 af[2][MT], bfr[2][NT];
            read_frags(buf, 0, af[0], bfr[0]);
#pragma unroll
            for (int kk = 0; kk < kBK / 16; ++kk) {
                if (kk + 1 < kBK / 16) read_frags(buf, kk + 1, af[(kk + 1) & 1], bfr[(kk + 1) & 1]);
                if (s + 1 < S && kk < 2) {   // early, so the loads land before the stage ends
#pragma unroll
                    for (int q = 4 * kk; q < 4 * kk + 4 && q < IW; ++q) dma(s + 1, buf ^ 1, q);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < NT; ++j) acc[i][j] = mfma32_bf16(af[kk & 1][i], bfr[kk & 1][j], acc[i][j]);
                __builtin_amdgcn_sched_barrier(0);
            }
            wait_vmcnt<0>();
            __syncthreads();
        }
    }

    // accumulator element r of tile (i, j): row 8(r/4) + 4(lane/32) + r%4, column lane%32
    if constexpr (!C_F32) {
        if (g.vt) {
            // kv_b value form: a lane's 4 consecutive rows of a value column
            // are 4 consecutive positions of one vt feature row (8 bytes)
            // the column (and so the target) depends on j only: one division per j
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int n = n0 + (BN / 2) * wn + 32 * j + (l & 31);
                const int hq = n / g.vt_period, c = n - hq * g.vt_period;
                const int64_t frow = (int64_t)hq * (g.vt_period - g.vt_from) + (c - g.vt_from);
#pragma unroll
                for (int i = 0; i < MT; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int mb = m0 + 64 * wm + 32 * i + 8 * q + 4 * (l >> 5);
                        if (c >= g.vt_from) {
                            if (mb >= g.vt_np) continue;
                            uint32_t two[2];
#pragma unroll
                            for (int e = 0; e < 2; ++e) {
                                const float lo = mb + 2 * e < g.M ? acc[i][j][4 * q + 2 * e] : 0.f;
                                const float hi = mb + 2 * e + 1 < g.M ? acc[i][j][4 * q + 2 * e + 1] : 0.f;
                                two[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
                                         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
                            }
                            const int k = mb & 31;
                            *reinterpret_cast<u32x2*>(g.vt + frow * g.vt_np + (mb - k) + 8 * ((k & 15) >> 2) + 4 * (k >> 4)) =
                                u32x2{two[0], two[1]};
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                if (mb + e >= g.M) continue;
                                const uint32_t u = __float_as_uint(acc[i][j][4 * q + e]);
                                static_cast<uint16_t*>(g.C)[(int64_t)(mb + e) * g.ldc + n] =
                                    (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                            }
                        }
                    }
                }
            }
            return;
        }
    }
    // Non-temporal stores: the output is not read again by this launch, and
    // streaming it past the L2 let the stores overlap the MFMAs far better
    // (o_proj 806 -> 706 us, q absorption 151 -> 113 us, up-projection
    // 173 -> 150 us).  The kv_b value form above keeps ordinary stores: its
    // scattered 8-byte pieces took twice as long when streamed.
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
            if (m >= g.M) continue;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int n = n0 + (BN / 2) * wn + 32 * j + (l & 31);
                const int64_t off = z * g.c_batch + (int64_t)m * g.ldc + n;
                if constexpr (C_F32) {
                    __builtin_nontemporal_store(acc[i][j][r], static_cast<float*>(g.C) + off);
                } else {
                    const uint32_t u = __float_as_uint(acc[i][j][r]);
                    __builtin_nontemporal_store((uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16),
                                                static_cast<uint16_t*>(g.C) + off);
                }
            }
        }
    }
}

// dst[r, dst_col0 + c] = src[r, src_col0 + c] for c < ncols, rows r < rows,
// in 16-byte chunks (ncols, the column offsets and the row strides are
// multiples of 8 bf16).  One thread per chunk.
__global__ __launch_bounds__(256) void copy_cols_kernel(const uint16_t* __restrict__ src, int64_t src_ld, int src_col0,
                                                        uint16_t* __restrict__ dst, int64_t dst_ld, int dst_col0,
                                                        int64_t rows, int ncols) {
    const int cpr = ncols / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= rows * cpr) return;
    const int64_t r = gid / cpr;
    const int c = (int)(gid - r * cpr) * 8;
    *reinterpret_cast<u32x4*>(dst + r * dst_ld + dst_col0 + c) = ldg16(src + r * src_ld + src_col0 + c);
}

// wkT[h, d, c] = w[h*(Dn+Dv) + c, d] for c < Dn, d < Dl: the key block of
// each head transposed, through a 64 x 64 LDS tile (rows padded by one
// element so the column reads do not conflict).  Block (d tile, c tile, h).
__global__ __launch_bounds__(256) void absorb_weight_kernel(const uint16_t* __restrict__ w, int Dn, int Dv, int Dl,
                                                            uint16_t* __restrict__ wkT) {
    __shared__ uint16_t tile[64][65];
    const int d0 = blockIdx.x * 64, c0 = blockIdx.y * 64, h = blockIdx.z;
    const int64_t C = Dn + Dv;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) {   // tile row r: key row c0 + r, columns d0..d0+63
        const int c = c0 + r, d = d0 + tx;
        tile[r][tx] = (c < Dn && d < Dl) ? w[((int64_t)h * C + c) * Dl + d] : (uint16_t)0;
    }
    __syncthreads();
    for (int r = ty; r < 64; r += 4) {   // output row d0 + r, columns c0..c0+63
        const int d = d0 + r, c = c0 + tx;
        if (d < Dl && c < Dn) wkT[((int64_t)h * Dl + d) * Dn + c] = tile[tx][r];
    }
}

}  // namespace

hipError_t launch_copy_cols(const uint16_t* src, int64_t src_ld, int src_col0, uint16_t* dst, int64_t dst_ld,
                            int dst_col0, int64_t rows, int ncols, hipStream_t s) {
    if (rows <= 0 || ncols <= 0) return hipSuccess;
    if (ncols % 8 || src_ld % 8 || dst_ld % 8 || src_col0 % 8 || dst_col0 % 8) return hipErrorInvalidValue;
    const int64_t n = rows * (ncols / 8);
    hipLaunchKernelGGL(copy_cols_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, src_ld, src_col0,
                       dst, dst_ld, dst_col0, rows, ncols);
    return hipGetLastError();
}

hipError_t launch_absorb_weight(const uint16_t* w, int H, int Dn, int Dv, int Dl, uint16_t* wkT, hipStream_t s) {
    if (H <= 0 || Dn <= 0 || Dl <= 0) return hipSuccess;
    const dim3 grid((unsigned)((Dl + 63) / 64), (unsigned)((Dn + 63) / 64), (unsigned)H);
    hipLaunchKernelGGL(absorb_weight_kernel, grid, dim3(256), 0, s, w, Dn, Dv, Dl, wkT);
    return hipGetLastError();
}

hipError_t launch_value_up_proj(const GemmArgs& g, int batch, hipStream_t s) {
    if (g.M <= 0 || batch <= 0) return hipSuccess;
    if (g.N != 256 || g.K % kBK != 0) return hipErrorInvalidValue;
    const dim3 grid((g.M + kBM - 1) / kBM, 1, batch);
    hipLaunchKernelGGL((gemm_nt_kernel<true, false, 256>), grid, dim3(kGemmThreads), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_o_proj(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0) return hipSuccess;
    if (g.N % 192 != 0 || g.K % kBK != 0) return hipErrorInvalidValue;
    // operand rows are addressed with 32-bit byte offsets
    if ((int64_t)g.M * g.lda * 2 >= (1ll << 32) || (int64_t)g.N * g.ldb * 2 >= (1ll << 32)) return hipErrorInvalidValue;
    const int tiles = (g.M + kBM - 1) / kBM * (g.N / 192);
    const dim3 grid((unsigned)(8 * ((tiles + 7) / 8)), 1, 1);
    hipLaunchKernelGGL((gemm_nt_kernel<false, true, 192>), grid, dim3(kGemmThreads), 0, s, g);
    return hipGetLastError();
}

// Query absorption: per head z, C = q_nope (rows of A) times the head's
// transposed key block (B, Dl rows of Dn), written into the first Dl columns
// of the head's absorbed query; the rope columns are copied by
// copy_cols_kernel.
hipError_t launch_q_absorb(const GemmArgs& g, int batch, hipStream_t s) {
    if (g.M <= 0 || batch <= 0) return hipSuccess;
    if (g.N % 256 != 0 || g.K % kBK != 0) return hipErrorInvalidValue;
    if ((int64_t)g.M * g.lda * 2 >= (1ll << 32) || (int64_t)g.N * g.ldb * 2 >= (1ll << 32)) return hipErrorInvalidValue;
    const int tiles = (g.M + kBM - 1) / kBM * (g.N / 256);
    const dim3 grid((unsigned)(8 * ((tiles + 7) / 8)), 1, (unsigned)batch);
    hipLaunchKernelGGL((gemm_nt_kernel<false, false, 256>), grid, dim3(kGemmThreads), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_kv_b_proj(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0) return hipSuccess;
    if (g.N % 256 != 0 || g.K % kBK != 0) return hipErrorInvalidValue;
    if ((int64_t)g.M * g.lda * 2 >= (1ll << 32) || (int64_t)g.N * g.ldb * 2 >= (1ll << 32)) return hipErrorInvalidValue;
    const int tiles = (g.M + kBM - 1) / kBM * (g.N / 256);
    const dim3 grid((unsigned)(8 * ((tiles + 7) / 8)), 1, 1);
    hipLaunchKernelGGL((gemm_nt_kernel<false, false, 256>), grid, dim3(kGemmThreads), 0, s, g);
    return hipGetLastError();
}

}  // namespace dsa
