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
//  - one block = one head x 128 queries (8 waves x 16 queries, two waves
//    per SIMD, so that one wave's MFMAs run beside the other's softmax,
//    LDS reads and DMA issue); the keys
//    stream in 64-key tiles through two LDS buffers filled by LDS-DMA
//    (global_load_lds), so key and value rows never pass through VGPRs.  A
//    tile holds the no-rope keys [64][Dn], the rope keys [64][Dr], the
//    values [64][Dv] and the block's 64-key mask words [128][2];
//  - scores S^T = K Q^T on bf16 MFMA 16x16x32 (each wave keeps its queries
//    in registers for the whole loop), an fp32 online softmax whose
//    reference maximum only moves when a score clears it by kLazy (log2
//    units), P in fp16, O^T += V^T P^T on fp16 MFMA.  The values come in one
//    of two forms: the kv_b output's bf16 columns, read transposed
//    (ds_read_b64_tr_b16) and converted to fp16 in registers; or a
//    feature-major fp16 copy vt [H][Dv][Np] (values_to_vt_kernel, or the
//    kv_b product directly), read as plain 16-byte fragments.  The fp16 form
//    takes the conversion (a third of the loop's vector instructions) out of
//    the loop, and its reads are conflict-free b128 reads (8% faster than
//    the transposing reads);
//  - the blocks of one head are consecutive in one XCD's share of the
//    dispatch order, so that head's keys and values stream through that
//    XCD's L2 once for all its query blocks.
// Numerics: bf16 products summed in fp32; P rounded to fp16 (relative 2^-11)
// and V converted bf16 -> fp16 (exact for |v| in [2^-14, 65504]; smaller
// magnitudes become fp16 subnormals, error at most 2^-25).
#include "dsa_kernels.h"

#include <math.h>

namespace dsa {
namespace {

constexpr int kDTK = 64;      // keys per tile
constexpr int kDQB = 128;     // queries per block
constexpr int kDNW = 8;       // waves per block
constexpr int kDQW = kDQB / kDNW;   // queries per wave (16)
constexpr int kDNT = 64 * kDNW;
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

__device__ inline uint32_t pack2_f16(float a, float b) { return pack_f16_rne(a, b); }

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
    static_assert((kDTK * CN / 64) % kDNW == 0 && (kDTK * CR / 64) % kDNW == 0 && (kDTK * CV / 64) % kDNW == 0,
                  "each wave issues a whole share of every region");
    static constexpr int KS = DQ / 32, KSN = DN / 32;             // score k-steps, no-rope first
    static constexpr int FB = DV / 16;                            // 16-feature output blocks
    static constexpr int SWN = swz_mask(CN, 8), SWR = swz_mask(CR, 8), SWV = swz_mask(CV, 16);
    struct Buf {
        u32x4 kn[kDTK * CN];
        u32x4 kr[kDTK * CR];
        u32x4 v[kDTK * CV];      // [key][Dv] (bf16 form) or [Dv][key] (vt form): same size
        uint32_t m[kDQB * 2];    // [query of the block][2 words]
    };
};

// VT: the values come from vt [H][Dv][Np] fp16 (Np = N rounded up to 64,
// zero past N): feature row f of head h holds key k at position
// 32 (k / 32) + vt_pos(k % 32), the order in which the P fragments list a
// 32-key step's keys (lane group g: keys 4g..4g+3, then 16+4g..16+4g+3), so
// that one 16-byte read is one MFMA operand.  Otherwise the values are the
// kvb columns Dn..Dn+Dv-1 in bf16.
template <int DN, int DR, int DV, bool VT>
__global__ __launch_bounds__(kDNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dense_attn_kernel(DenseArgs a) {
    using C = DenseShape<DN, DR, DV>;
    __shared__ __attribute__((aligned(16))) typename C::Buf buf[2];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 4, c16 = l & 15;

    // block -> (head, query block): XCD x (blocks b with b % 8 == x) takes a
    // contiguous run of heads; heavier (later) query blocks first
    const int nqb = (a.L + kDQB - 1) / kDQB;
    const int total = nqb * a.H;
    const int b = blockIdx.x;
    const int lin = (total % 8 == 0) ? (b % 8) * (total / 8) + b / 8 : b;
    const int h = lin / nqb;
    const int q0 = (nqb - 1 - lin % nqb) * kDQB;
    const int qlast = min(q0 + kDQB, a.L) - 1;
    const int nkeys = min(a.N, a.q_start + qlast + 1);      // keys after the last query are never visible
    const int ntiles = (nkeys + kDTK - 1) / kDTK;

    // this lane's query (B operand: query c16 of the wave, dims 8g..8g+7 of each k-step)
    u32x4 qf[C::KS];
    {
        const int qq = min(q0 + kDQW * w + c16, a.L - 1);
        const uint16_t* qr = a.q + ((int64_t)qq * a.H + h) * C::DQ + 8 * g;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) qf[ks] = ldg16(qr + 32 * ks);
    }

    // LDS-DMA of tile t into buffer bi.  Instruction n of a region writes its
    // 64 consecutive chunk slots; slot P is row P / chunks, stored chunk
    // P % chunks, which holds logical chunk (P % chunks) ^ swizzle(row).
    // Rows past the last key repeat it (their mask bits are 0).
    const uint32_t rs_kvb = (uint32_t)a.H * C::DKV * 2u, rs_kv = (uint32_t)a.kv_cols * 2u;
    constexpr int IN = kDTK * C::CN / 64 / kDNW, IR = kDTK * C::CR / 64 / kDNW,
                  IV = kDTK * C::CV / 64 / kDNW;   // instructions per wave and region
    uint32_t off[IN + IR + IV];   // byte offset of this lane's chunk from the tile's first row
    int row[IN + IR + IV];        // ... and its tile row
#pragma unroll
    for (int n = 0; n < IN + IR + IV; ++n) {
        const int ch = n < IN ? C::CN : n < IN + IR ? C::CR : C::CV;
        const int i = w * (n < IN ? IN : n < IN + IR ? IR : IV) + (n < IN ? n : n < IN + IR ? n - IN : n - IN - IR);
        const int P = 64 * i + l, r = P / ch;
        const int x = n < IN ? swz_key(r & 15) & C::SWN : n < IN + IR ? swz_key(r & 15) & C::SWR : swz_val(r & 15) & C::SWV;
        row[n] = r;
        off[n] = (uint32_t)r * (n < IN + IR && n >= IN ? rs_kv : rs_kvb) + 16u * ((P % ch) ^ x);
    }
    // vt form: the lane's chunk of each value instruction, from its tile's first key
    uint32_t voff[IV];
#pragma unroll
    for (int n = 0; n < IV; ++n) {
        const int P = 64 * (w * IV + n) + l, r = P / 8;
        voff[n] = (uint32_t)r * (uint32_t)a.Np * 2u + 16u * ((P % 8) ^ (swz_key(r & 15) & 7));
    }
    auto issue = [&](int t, int bi) {
        typename C::Buf& B = buf[bi];
        const int k0 = t * kDTK;
        const uint16_t* kvb_t = a.kvb + ((int64_t)k0 * a.H + h) * C::DKV;
        const uint16_t* kv_t = a.kv + (int64_t)k0 * a.kv_cols + a.rope_col;
        // the tile reaches past the last key: its extra rows repeat the last key
        const bool clamp = k0 + kDTK > a.N;
        const int jmax = a.N - 1 - k0;
        auto src_off = [&](int n, uint32_t rs) {
            return clamp && row[n] > jmax ? off[n] - (uint32_t)(row[n] - jmax) * rs : off[n];
        };
#pragma unroll
        for (int n = 0; n < IN; ++n)
            gather16_to_lds(kvb_t, src_off(n, rs_kvb), lds_addr(&B.kn[64 * (w * IN + n)]));
#pragma unroll
        for (int n = 0; n < IR; ++n)
            gather16_to_lds(kv_t, src_off(IN + n, rs_kv), lds_addr(&B.kr[64 * (w * IR + n)]));
        if constexpr (VT) {
            // feature rows of 64 keys (128 B, 8 chunks), chunk XOR as for the rope rows
            const uint16_t* vbase = a.vt + (int64_t)h * DV * a.Np + k0;
#pragma unroll
            for (int n = 0; n < IV; ++n)
                gather16_to_lds(vbase, voff[n], lds_addr(&B.v[64 * (w * IV + n)]));
        } else {
#pragma unroll
            for (int n = 0; n < IV; ++n)
                gather16_to_lds(kvb_t + DN, src_off(IN + IR + n, rs_kvb), lds_addr(&B.v[64 * (w * IV + n)]));
        }
        // mask words: lane l < 32 -> query 16w + l / 2 of the block, word l % 2 of the tile
        const uint32_t* mb = a.mask + (int64_t)q0 * a.W + k0 / 32;
        const int qi = min(kDQW * w + (l >> 1), a.L - 1 - q0);
        if (l < 2 * kDQW) load4_to_lds(mb, (uint32_t)(qi * a.W + (l & 1)) * 4u, lds_addr(&B.m[2 * kDQW * w]));
    };

    f32x4 o[C::FB];
#pragma unroll
    for (int f = 0; f < C::FB; ++f) o[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the reference maximum starts finite, so that exp2(-inf - mref) = 0 for a
    // masked-out key even before the first visible one
    constexpr float kStart = -1e30f;
    float mref = kStart, lsum = 0.f;

    // per-lane LDS read offsets
    const int xn = swz_key(c16) & C::SWN, xr = swz_key(c16) & C::SWR, xr8 = swz_key(c16) & 7;
    const int trow = 4 * g + (c16 >> 2);
    const int vx = (swz_val(trow) & C::SWV) ^ ((c16 >> 1) & 1);
    const int vrow = trow * C::CV * 16 + 8 * (c16 & 1);

    if (ntiles > 0) issue(0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int bi = t & 1;
        const typename C::Buf& B = buf[bi];

        // scores: s[kb] holds keys 16kb + 4g + i of query c16
        f32x4 s[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
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
            for (int kb = 0; kb < 4; ++kb) s[kb] = mfma16_bf16(ka[kb], qf[ks], s[kb]);
        }

        // mask, online softmax, P^T fragments (keys 4g..4g+3 and 16+4g..16+4g+3
        // of each 32-key step, matching the transposed value read)
        u32x4 pf[2];
        {
            const uint32_t* mw = &B.m[2 * (kDQW * w + c16)];
            float x[4][4];
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const uint32_t nib = mw[kb >> 1] >> (16 * (kb & 1) + 4 * g);   // this lane's 4 keys
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // 0 for a visible key, -inf (bits 0xff800000) for a masked one
                    const float bias = __uint_as_float(((nib >> i) & 1u) ? 0u : 0xff800000u);
                    x[kb][i] = fmaf(s[kb][i], a.scale_log2, bias);
                    mt = fmaxf(mt, x[kb][i]);
                }
            }
            mt = max_q4(mt);
            const bool up = mt > mref + kDLazy;
            if (__ballot(up)) {   // wave-uniform; rare after the first tiles
                const float mn = up ? mt : mref;
                const float alpha = up ? __builtin_amdgcn_exp2f(mref - mn) : 1.f;
                mref = mn;
                lsum *= alpha;
#pragma unroll
                for (int f = 0; f < C::FB; ++f) o[f] *= alpha;
            }
            float p[4][4];
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[kb][i] = __builtin_amdgcn_exp2f(x[kb][i] - mref);
                    ps += p[kb][i];
                }
            lsum += ps;
#pragma unroll
            for (int st = 0; st < 2; ++st)
                pf[st] = u32x4{pack2_f16(p[2 * st][0], p[2 * st][1]), pack2_f16(p[2 * st][2], p[2 * st][3]),
                               pack2_f16(p[2 * st + 1][0], p[2 * st + 1][1]),
                               pack2_f16(p[2 * st + 1][2], p[2 * st + 1][3])};
        }

        // the next tile's DMA goes out here, after this tile's score reads: an
        // LDS read that a wave issues behind its own LDS-DMA loads waits on
        // them, and the score reads are the larger share (issued first, at
        // the top of the tile, the kernel took 12% longer)
        if (t + 1 < ntiles) issue(t + 1, bi ^ 1);

        // O^T[feature][query] += V^T P^T
        const unsigned char* vt = reinterpret_cast<const unsigned char*>(B.v);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
            for (int f = 0; f < C::FB; ++f) {
                u32x4 av;
                if constexpr (VT) {
                    av = *reinterpret_cast<const u32x4*>(vt + (16 * f + c16) * 128 + 16 * ((4 * st + g) ^ xr8));
                } else {
                    const int off = (32 * st) * C::CV * 16 + vrow + 16 * ((2 * f) ^ vx);
                    const u32x2 v0 = bf16x4_f16x4(read_tr16(vt + off));
                    const u32x2 v1 = bf16x4_f16x4(read_tr16(vt + off + 16 * C::CV * 16));
                    av = u32x4{v0[0], v0[1], v1[0], v1[1]};
                }
                o[f] = mfma16_f16(av, pf[st], o[f]);
            }
        }
        wait_vmcnt<0>();     // this wave's share of tile t+1 has landed
        __syncthreads();     // ... and everyone's; buffer bi is free again
    }

    // normalise and store: lane holds features 16f + 4g .. +3 of query c16
    {
        const float tot = sum_q4(lsum);
        const float inv = tot > 0.f ? 1.f / tot : 0.f;
        const int qq = q0 + kDQW * w + c16;
        if (qq < a.L) {
            float* orow = a.out + ((int64_t)qq * a.H + h) * DV + 4 * g;
#pragma unroll
            for (int f = 0; f < C::FB; ++f) *reinterpret_cast<f32x4*>(orow + 16 * f) = o[f] * inv;
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
    auto mark = [&](int t, int j) {
        if (t < c && j >= 0 && j < a.N && j <= p) atomicOr(&bits[j >> 5], 1u << (j & 31));
    };
    if ((a.top_k & 3) == 0) {
        // four ids per 16-byte load (rows start 16-byte aligned), two loads
        // in flight per thread before any atomic; ids past c are read (they
        // lie in the row) and ignored
        for (int t0 = 4 * (int)threadIdx.x; t0 < c; t0 += 2 * 4 * 256) {
            const int t1 = t0 + 4 * 256;
            const int4 x = *reinterpret_cast<const int4*>(sel + t0);
            const int4 y = t1 < c ? *reinterpret_cast<const int4*>(sel + t1) : int4{-1, -1, -1, -1};
            mark(t0, x.x); mark(t0 + 1, x.y); mark(t0 + 2, x.z); mark(t0 + 3, x.w);
            mark(t1, y.x); mark(t1 + 1, y.y); mark(t1 + 2, y.z); mark(t1 + 3, y.w);
        }
    } else {
        for (int t = threadIdx.x; t < c; t += 256) mark(t, sel[t]);
    }
    __syncthreads();
    uint32_t* row = a.mask + (int64_t)i * a.W;
    for (int k = threadIdx.x; k < a.W; k += 256) row[k] = bits[k];
}

// kvb's value columns (bf16) -> vt [H][Dv][Np] fp16, round to nearest even
// (exact for |v| in [2^-14, 65504]; larger magnitudes become infinities),
// keys past N zero.  Block = one head x 64 keys: the 64 value rows go through
// LDS and come out as 16-byte pieces of the feature rows.  Position p of a
// 32-key group holds key 4(p / 8) + (p % 4) + 16((p / 4) % 2).
template <int DV>
__global__ __launch_bounds__(256) void values_to_vt_kernel(const uint16_t* kvb, int N, int H, int dn, int Np,
                                                           uint16_t* vt) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][DV + 8];   // [key][feature], rows padded by 16 B
    const int h = blockIdx.y, k0 = blockIdx.x * 64, tid = threadIdx.x;
    const int64_t rowlen = (int64_t)H * (dn + DV);
    for (int i = tid; i < 64 * DV / 8; i += 256) {
        const int k = i / (DV / 8), c = i % (DV / 8);
        u32x4 x = {0u, 0u, 0u, 0u};
        if (k0 + k < N) x = ldg16(kvb + (int64_t)(k0 + k) * rowlen + (int64_t)h * (dn + DV) + dn + 8 * c);
        *reinterpret_cast<u32x4*>(&tile[k][8 * c]) = x;
    }
    __syncthreads();
    for (int i = tid; i < DV * 8; i += 256) {   // piece: feature f, tile positions 8q..8q+7
        const int f = i / 8, q = i % 8;
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            uint32_t two = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int p = 8 * (q & 3) + j + e;                              // position in the group
                const int k = 32 * (q >> 2) + 4 * (p >> 3) + (p & 3) + 16 * ((p >> 2) & 1);
                const _Float16 x = (_Float16)__uint_as_float((uint32_t)tile[k][f] << 16);
                two |= (uint32_t)__builtin_bit_cast(uint16_t, x) << (16 * e);
            }
            o[j / 2] = two;
        }
        // streamed past the L2 (read by a later launch): 116 -> 103 us at 8k keys
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(vt + ((int64_t)h * DV + f) * Np + k0 + 8 * q));
    }
}

}  // namespace

hipError_t launch_values_to_vt(const uint16_t* kvb, int N, int H, int dn, int dv, int Np, uint16_t* vt,
                               hipStream_t s) {
    if (N <= 0) return hipSuccess;
    const dim3 grid((unsigned)(Np / 64), (unsigned)H);
    if (dv == 256) hipLaunchKernelGGL(values_to_vt_kernel<256>, grid, dim3(256), 0, s, kvb, N, H, dn, Np, vt);
    else if (dv == 64) hipLaunchKernelGGL(values_to_vt_kernel<64>, grid, dim3(256), 0, s, kvb, N, H, dn, Np, vt);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_selection_mask(const MaskArgs& a, hipStream_t s) {
    if (a.L <= 0) return hipSuccess;
    hipLaunchKernelGGL(selection_mask_kernel, dim3((unsigned)a.L), dim3(256), (size_t)a.W * 4u, s, a);
    return hipGetLastError();
}

hipError_t launch_dense_attn(int shape_id, const DenseArgs& a, hipStream_t s) {
    const bool values_f16 = a.vt != nullptr;
    if (a.L <= 0 || a.N <= 0) return hipSuccess;
    const int nqb = (a.L + kDQB - 1) / kDQB;
    const dim3 grid((unsigned)(nqb * a.H)), block(kDNT);
    if (shape_id == 0) {
        if (values_f16) hipLaunchKernelGGL((dense_attn_kernel<192, 64, 256, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((dense_attn_kernel<192, 64, 256, false>), grid, block, 0, s, a);
    } else {
        if (values_f16) hipLaunchKernelGGL((dense_attn_kernel<64, 64, 64, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((dense_attn_kernel<64, 64, 64, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace dsa
