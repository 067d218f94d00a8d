// dense.hip - dense masked attention in the non-absorbed form, on gfx950.
//
// exo PR #2539, Prefill section (dense attention in one product): below
// 8192 keys of context each head scores its 192 no-rope and 64 rope
// dimensions in one 256-wide product under a boolean mask, instead of
// gathering the selected latent rows.  The pipeline trace's config line
// gives the widths (qk_nope 192, qk_rope 64, v_head_dim 256); its section 4
// splits the kv_b output per head into the no-rope key and the value, and
// the rope key is the one k_pe of the cache row, shared by all heads.  The
// mask is the query's selection, limited to causal keys.
//
// Layout and schedule:
//  - one block = one head x 128 queries (4 waves x 32 queries); the keys
//    stream in 64-key tiles through two LDS buffers filled by LDS-DMA
//    (global_load_lds), so key and value rows never pass through VGPRs.  A
//    tile holds the no-rope keys [64][Dn], the rope keys [64][Dr], the
//    values [64][Dv] and the block's 64-key mask words [128][2];
//  - scores S^T = K Q^T on bf16 MFMA 16x16x32 (each wave keeps its queries
//    in registers for the whole loop), an fp32 online softmax whose
//    reference maximum only moves when a score clears it by kLazy (log2
//    units), P in fp16, O^T += V^T P^T on fp16 MFMA with V read transposed
//    (ds_read_b64_tr_b16) and converted to fp16 in registers;
//  - the blocks of one head are consecutive in one XCD's share of the
//    dispatch order, so that head's keys and values stream through that
//    XCD's L2 once for all its query blocks.
// Numerics: bf16 products summed in fp32; P rounded to fp16 (relative 2^-11)
// and V converted bf16 -> fp16 (exact for |v| in [2^-14, 65504]).
#include "dsa_kernels.h"

#include <math.h>

namespace dsa {
namespace {

constexpr int kDTK = 64;      // keys per tile
constexpr int kDQB = 128;     // queries per block
constexpr int kDNT = 256;     // threads per block (4 waves)
constexpr float kDLazy = 8.f;

// Chunk XORs of LDS tile rows (rows 16 apart share one).  Value rows (512 B)
// take the map bit 0 -> 3, bit 1 -> 4, bit 2 -> 8, bit 3 -> 10, which keeps
// the transposed value read free of bank conflicts; no-rope key rows (384 B)
// and rope key rows (128 B) take bit 1 -> 4, bit 3 -> 2, which keeps the score
// read (lane l: row l & 15, chunk 4k + l / 16) free of them for both strides.
// Each map is masked to the chunks of its row.
__device__ inline int swz_val(int r) {
    return ((r & 1) ? 3 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 8 : 0) ^ ((r & 8) ? 10 : 0);
}
__device__ inline int swz_key(int r) { return ((r & 2) ? 4 : 0) ^ ((r & 8) ? 2 : 0); }

constexpr int swz_mask(int chunks, int cap) {
    return ((chunks & -chunks) < cap ? (chunks & -chunks) : cap) - 1;
}

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lds_bf16x4_t;

__device__ inline u32x2 read_tr16(const unsigned char* p) {
    const DSA_LDS lds_bf16x4_t* a = (const DSA_LDS lds_bf16x4_t*)(p);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((DSA_LDS lds_bf16x4_t*)a));
}

__device__ inline uint32_t pack2_f16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// 4 bf16 -> 4 fp16 (exact in the fp16 normal range)
__device__ inline u32x2 bf16x4_f16x4(const u32x2& d) {
    return u32x2{pack2_f16(__uint_as_float(d[0] << 16), __uint_as_float(d[0] & 0xFFFF0000u)),
                 pack2_f16(__uint_as_float(d[1] << 16), __uint_as_float(d[1] & 0xFFFF0000u))};
}

// max / sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes of a query)
__device__ inline float max_q4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_q4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int DN, int DR, int DV>
struct DenseShape {
    static_assert(DN % 32 == 0 && DR % 32 == 0 && DV % 16 == 0, "head widths");
    static constexpr int DQ = DN + DR, DKV = DN + DV;
    static constexpr int CN = DN / 8, CR = DR / 8, CV = DV / 8;   // 16-byte chunks per row
    static_assert(CN % 4 == 0 && CR % 4 == 0 && CV % 4 == 0, "each wave issues a whole share of every region");
    static constexpr int KS = DQ / 32, KSN = DN / 32;             // score k-steps, no-rope first
    static constexpr int FB = DV / 16;                            // 16-feature output blocks
    static constexpr int SWN = swz_mask(CN, 8), SWR = swz_mask(CR, 8), SWV = swz_mask(CV, 16);
    struct Buf {
        u32x4 kn[kDTK * CN];
        u32x4 kr[kDTK * CR];
        u32x4 v[kDTK * CV];
        uint32_t m[kDQB * 2];    // [wave][query of the wave][2 words]
    };
};

template <int DN, int DR, int DV>
__global__ __launch_bounds__(kDNT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void dense_attn_kernel(DenseArgs a) {
    using C = DenseShape<DN, DR, DV>;
    __shared__ __attribute__((aligned(16))) typename C::Buf buf[2];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;

    // block -> (head, query block): XCD x (blocks b with b % 8 == x) takes a
    // contiguous run of heads; heavier (later) query blocks first
    const int nqb = (a.L + kDQB - 1) / kDQB;
    const int total = nqb * a.H;
    const int b = blockIdx.x;
    const int v = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
    const int h = v / nqb;
    const int q0 = (nqb - 1 - v % nqb) * kDQB;
    const int qlast = min(q0 + kDQB, a.L) - 1;
    const int nkeys = min(a.N, a.q_start + qlast + 1);      // keys after the last query are never visible
    const int ntiles = (nkeys + kDTK - 1) / kDTK;

    // this lane's queries (B operand: query c16 of each 16-query half, dims 8g..8g+7 of each k-step)
    u32x4 qf[2][C::KS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qq = min(q0 + 32 * w + 16 * qb + c16, a.L - 1);
        const uint16_t* qr = a.q + ((int64_t)qq * a.H + h) * C::DQ + 8 * g;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qf[qb][ks] = ldg16(qr + 32 * ks);
    }

    // LDS-DMA of tile t into buffer bi.  Instruction n of a region writes its
    // 64 consecutive chunk slots; slot P is row P / chunks, stored chunk
    // P % chunks, which holds logical chunk (P % chunks) ^ swizzle(row).
    // Rows past the last key repeat it (their mask bits are 0).
    const uint32_t rs_kvb = (uint32_t)a.H * C::DKV * 2u, rs_kv = (uint32_t)a.kv_cols * 2u;
    auto issue = [&](int t, int bi) {
        typename C::Buf& B = buf[bi];
        const int k0 = t * kDTK;
        const int jmax = a.N - 1 - k0;
        const uint16_t* kvb_t = a.kvb + ((int64_t)k0 * a.H + h) * C::DKV;
        const uint16_t* kv_t = a.kv + (int64_t)k0 * a.kv_cols + a.rope_col;
#pragma unroll
        for (int n = 0; n < C::CN / 4; ++n) {
            const int i = w * (C::CN / 4) + n, P = 64 * i + l, r = P / C::CN;
            const int c = (P % C::CN) ^ (swz_key(r & 15) & C::SWN);
            gather16_to_lds(kvb_t, (uint32_t)min(r, jmax) * rs_kvb + 16u * c, lds_addr(&B.kn[64 * i]));
        }
#pragma unroll
        for (int n = 0; n < C::CR / 4; ++n) {
            const int i = w * (C::CR / 4) + n, P = 64 * i + l, r = P / C::CR;
            const int c = (P % C::CR) ^ (swz_key(r & 15) & C::SWR);
            gather16_to_lds(kv_t, (uint32_t)min(r, jmax) * rs_kv + 16u * c, lds_addr(&B.kr[64 * i]));
        }
#pragma unroll
        for (int n = 0; n < C::CV / 4; ++n) {
            const int i = w * (C::CV / 4) + n, P = 64 * i + l, r = P / C::CV;
            const int c = (P % C::CV) ^ (swz_val(r & 15) & C::SWV);
            gather16_to_lds(kvb_t + DN, (uint32_t)min(r, jmax) * rs_kvb + 16u * c, lds_addr(&B.v[64 * i]));
        }
        // mask words: lane l -> query 32w + l / 2 of the block, word l % 2 of the tile
        const uint32_t* mb = a.mask + (int64_t)q0 * a.W + k0 / 32;
        const int qi = min(32 * w + (l >> 1), a.L - 1 - q0);
        load4_to_lds(mb, (uint32_t)(qi * a.W + (l & 1)) * 4u, lds_addr(&B.m[64 * w]));
    };

    f32x4 o[C::FB][2];
#pragma unroll
    for (int f = 0; f < C::FB; ++f) o[f][0] = o[f][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mref[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};

    // per-lane LDS read offsets
    const int xn = swz_key(c16) & C::SWN, xr = swz_key(c16) & C::SWR;
    const int trow = 4 * g + (c16 >> 2);
    const int vx = (swz_val(trow) & C::SWV) ^ ((c16 >> 1) & 1);
    const int vrow = trow * C::CV * 16 + 8 * (c16 & 1);

    if (ntiles > 0) issue(0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int bi = t & 1;
        if (t + 1 < ntiles) issue(t + 1, bi ^ 1);
        const typename C::Buf& B = buf[bi];

        // scores: s[qb][kb] holds keys 16kb + 4g + i of query 16qb + c16
        f32x4 s[2][4];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            u32x4 ka[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int r = 16 * kb + c16;
                ka[kb] = ks < C::KSN ? B.kn[r * C::CN + ((4 * ks + g) ^ xn)]
                                     : B.kr[r * C::CR + ((4 * (ks - C::KSN) + g) ^ xr)];
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) s[qb][kb] = mfma16_bf16(ka[kb], qf[qb][ks], s[qb][kb]);
        }

        // mask, online softmax, P^T fragments (keys 4g..4g+3 and 16+4g..16+4g+3
        // of each 32-key step, matching the transposed value read)
        u32x4 pf[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const uint64_t mw = *reinterpret_cast<const uint64_t*>(&B.m[64 * w + 2 * (16 * qb + c16)]);
            float x[4][4];
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = (mw >> (16 * kb + 4 * g + i)) & 1u;
                    x[kb][i] = ok ? s[qb][kb][i] * a.scale_log2 : -INFINITY;
                    mt = fmaxf(mt, x[kb][i]);
                }
            mt = max_q4(mt);
            const bool up = mt > mref[qb] + kDLazy;
            if (__ballot(up)) {   // wave-uniform; rare after the first tiles
                const float mn = up ? mt : mref[qb];
                const float alpha = up ? __builtin_amdgcn_exp2f(mref[qb] - mn) : 1.f;
                mref[qb] = mn;
                lsum[qb] *= alpha;
#pragma unroll
                for (int f = 0; f < C::FB; ++f) o[f][qb] *= alpha;
            }
            float p[4][4];
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[kb][i] = x[kb][i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[kb][i] - mref[qb]);
                    ps += p[kb][i];
                }
            lsum[qb] += ps;
#pragma unroll
            for (int st = 0; st < 2; ++st)
                pf[qb][st] = u32x4{pack2_f16(p[2 * st][0], p[2 * st][1]), pack2_f16(p[2 * st][2], p[2 * st][3]),
                                   pack2_f16(p[2 * st + 1][0], p[2 * st + 1][1]),
                                   pack2_f16(p[2 * st + 1][2], p[2 * st + 1][3])};
        }

        // O^T[feature][query] += V^T P^T
        const unsigned char* vt = reinterpret_cast<const unsigned char*>(B.v);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int f = 0; f < C::FB; ++f) {
                const int off = (32 * st) * C::CV * 16 + vrow + 16 * ((2 * f) ^ vx);
                const u32x2 v0 = bf16x4_f16x4(read_tr16(vt + off));
                const u32x2 v1 = bf16x4_f16x4(read_tr16(vt + off + 16 * C::CV * 16));
                const u32x4 av = {v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) o[f][qb] = mfma16_f16(av, pf[qb][st], o[f][qb]);
            }
        }
        wait_vmcnt<0>();     // this wave's share of tile t+1 has landed
        __syncthreads();     // ... and everyone's; buffer bi is free again
    }

    // normalise and store: lane holds features 16f + 4g .. +3 of query 16qb + c16
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float tot = sum_q4(lsum[qb]);
        const float inv = tot > 0.f ? 1.f / tot : 0.f;
        const int qq = q0 + 32 * w + 16 * qb + c16;
        if (qq < a.L) {
            float* orow = a.out + ((int64_t)qq * a.H + h) * DV + 4 * g;
#pragma unroll
            for (int f = 0; f < C::FB; ++f) *reinterpret_cast<f32x4*>(orow + 16 * f) = o[f][qb] * inv;
        }
    }
}

// One block per query row: the row's bits are set in LDS, then written out.
__global__ __launch_bounds__(256) void selection_mask_kernel(MaskArgs a) {
    extern __shared__ uint32_t bits[];
    const int i = blockIdx.x;
    for (int k = threadIdx.x; k < a.W; k += 256) bits[k] = 0u;
    __syncthreads();
    const int c = min(max(a.count[i], 0), a.top_k);
    const int p = a.q_start + i;
    const int32_t* sel = a.idx + (int64_t)i * a.top_k;
    for (int t = threadIdx.x; t < c; t += 256) {
        const int j = sel[t];
        if (j >= 0 && j < a.N && j <= p) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    uint32_t* row = a.mask + (int64_t)i * a.W;
    for (int k = threadIdx.x; k < a.W; k += 256) row[k] = bits[k];
}

}  // namespace

hipError_t launch_selection_mask(const MaskArgs& a, hipStream_t s) {
    if (a.L <= 0) return hipSuccess;
    hipLaunchKernelGGL(selection_mask_kernel, dim3((unsigned)a.L), dim3(256), (size_t)a.W * 4u, s, a);
    return hipGetLastError();
}

hipError_t launch_dense_attn(int shape_id, const DenseArgs& a, hipStream_t s) {
    if (a.L <= 0 || a.N <= 0) return hipSuccess;
    const int nqb = (a.L + kDQB - 1) / kDQB;
    const dim3 grid((unsigned)(nqb * a.H)), block(kDNT);
    if (shape_id == 0) hipLaunchKernelGGL((dense_attn_kernel<192, 64, 256>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((dense_attn_kernel<32, 32, 64>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace dsa
