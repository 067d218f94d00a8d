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
// Design (one block = one query, or one chunk of a query's selection; one
// block per CU; at GLM shape eight waves, two per SIMD):
//  - producer waves (the first half) own the scores: wave w holds the query
//    fragments of heads 16w..16w+15, computes S^T = K Q^T for each tile on
//    v_mfma_f32_16x16x32_bf16 and runs the softmax; consumer waves (the
//    second half) own the output: consumer c accumulates features
//    128c..128c+127 of all heads.  The split keeps each wave under 256
//    registers, so a SIMD holds one wave of each kind and the matrix pipe
//    is fed by one while the other waits on LDS or runs its softmax.
//  - the selection is copied to LDS once (row ids plus a validity bitmap);
//    selected rows are then gathered 32 per tile straight into LDS with
//    global_load_lds_dwordx4 (16 bytes per lane, no registers) into a ring
//    of three tiles: while consumers read tile it and producers score tile
//    it+1, tile it+2 is in flight.  The consumers issue the whole gather:
//    handing a tile's loads to the CU's address unit holds the issuing wave
//    for hundreds of cycles, which the producers cannot spare.  The loads are issued from inline
//    assembly and waited for with explicit vmcnt counts: the compiler's own
//    wait insertion would drain every outstanding LDS load before each LDS
//    read.  A 1 KB latent row is one instruction with a scalar row address.
//    (A fourth tile in flight measured no faster.)
//  - a tile is stored in two row-major regions: the Dl latent columns (bf16,
//    or fp16 when the cache was converted once by latent_to_f16_kernel, which
//    removes the per-query conversion from the value path) and the bf16 rope
//    columns.  16-byte chunks are XOR-swizzled per row so that the score
//    reads (16 rows, one chunk) and the transposed value reads (4 rows,
//    2 chunks) run without bank conflicts (the map is at swz_lat).
//  - softmax in fp32 (base 2) with a lazy reference: the running maximum
//    used for the exponentials moves only when a score exceeds it by more
//    than 8 (probabilities stay <= 256), so the output rescale almost never
//    runs.  Producers publish probabilities (fp16, already in MFMA operand
//    layout) and rescale factors in LDS; one barrier per tile.
//  - values: O^T = V^T P^T on v_mfma_f32_16x16x32_f16; the value fragments
//    come from the row-major tile through ds_read_b64_tr_b16 (gfx950's
//    transposing read: within 16 lanes, lane i receives element i%4 of the
//    rows addressed by lanes i/4 + 4k) and are converted bf16 -> fp16 in
//    registers.  The key order of a producer lane's score accumulators is
//    exactly the consumer's probability operand.
//  - probabilities enter the value product as fp16 (11-bit significand,
//    rounded to nearest even, so the rounding is unbiased against the fp32
//    denominator): a bf16 probability operand alone would cost about 1.5e-3
//    relative error.
//    Latent values are exact in fp16 for |v| in [2^-14, 65504]; smaller ones
//    become fp16 subnormals (error at most 2^-25).
#include "dsa_kernels.h"

#include <math.h>

namespace dsa {
namespace {

constexpr int kTK = 32;        // keys per tile
constexpr int kRing = 3;       // tiles resident in LDS: the ring keeps kRing - 2 gathers in flight
constexpr float kLazy = 8.f;   // log2 headroom before the reference maximum moves
// Key fragments are read this many k-steps ahead of the MFMAs that use
// them.  Each read is pinned in program order by a compiler memory fence:
// left alone, the scheduler sinks the reads next to their MFMAs to save
// registers and every MFMA then waits out a full LDS latency.
constexpr int kKeyAhead = 2;

template <int NH, int DL, int DR>
struct AttnShape {
    static_assert(DL % 32 == 0 && DR % 8 == 0, "latent widths must be multiples of 32 / 8");
    static constexpr int NHB = (NH + 15) / 16;           // head blocks = producer waves = consumer waves
    static constexpr int NWAVE = 2 * NHB;
    static constexpr int NT = NWAVE * 64;
    static constexpr int DQK = DL + DR;
    static constexpr int DQKP = (DQK + 31) / 32 * 32;    // score K dim padded to the MFMA step
    static constexpr int KS = DQKP / 32;                 // score K steps
    static constexpr int KSL = DL / 32;                  // ... of them in the latent region
    static constexpr int FB = DL / 16;                   // value feature blocks
    static constexpr int FBW = FB / NHB;                 // value feature blocks per consumer
    static constexpr int CL = DL / 8;                    // 16-byte chunks of a latent row
    static constexpr int CR = (DQKP - DL) / 8;           // chunks of a rope row (with padding)
    static constexpr int CRD = DR / 8;                   // ... holding data
    static constexpr int LAT_B = kTK * CL * 16;          // latent region bytes
    static constexpr int TILE_B = LAT_B + kTK * CR * 16;
    static constexpr int IL = kTK * CL / 64;             // gather instructions, latent region
    static constexpr int IR = kTK * CR / 64;             // gather instructions, rope region
    static constexpr int NG = NHB;                       // gather waves (the consumers)
    static constexpr int ILW = IL / NG;                  // latent instructions per gather wave
    static constexpr int IRW = IR / NG;                  // rope instructions per gather wave
    static constexpr int LR = 64 / CL > 0 ? 64 / CL : 1; // rows per latent instruction
    static_assert((CL & (CL - 1)) == 0 && (CR & (CR - 1)) == 0, "row chunk counts must be powers of two");
    static_assert(64 % CL == 0 || CL == 64, "latent rows must pack whole instructions");
    static_assert(64 % CR == 0, "rope rows must pack whole instructions");
    static_assert(FB % NHB == 0 && IL % NG == 0 && IR % NG == 0 && kTK * CR % 64 == 0,
                  "work must split evenly");
};

// Chunk XOR of tile row r in the latent region (rows 16 apart share it) and
// in the rope region.  The latent XOR is linear in the bits of r (bit 0 -> 3,
// bit 1 -> 4, bit 2 -> 8, bit 3 -> 10), chosen by measurement: a 16-byte LDS
// read serves the wave 16 lanes at a time, and the lanes grouped together are
// not simply 16 consecutive ones, so the score read (lane l: row l & 15,
// chunk 4k + l / 16) needs chunks that differ across those groups.  With this
// map the score read runs at the conflict-free rate (182 B per clock per CU
// against 128 for the plain 2(r & 7) + (r >> 3 & 1) interleave), and the
// transposed value read (rows 4g..4g+3, two chunks) still hits 16 distinct
// chunks within each half wave (x >> 1 differs between rows 0-7 and between
// rows 8-15).
__device__ inline int swz_lat(int r) {
    return ((r & 1) ? 3 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 8 : 0) ^ ((r & 8) ? 10 : 0);
}
__device__ inline int swz_rope(int r) { return (r >> 1) & 7; }

__device__ inline uint32_t pack_f16(float a, float b) { return pack_f16_rne(a, b); }

// 4 bf16 (two dwords) -> 4 fp16
__device__ inline u32x2 bf16x4_to_f16x4(const u32x2& d) {
    u32x2 r;
    r[0] = pack_f16(__uint_as_float(d[0] << 16), __uint_as_float(d[0] & 0xFFFF0000u));
    r[1] = pack_f16(__uint_as_float(d[1] << 16), __uint_as_float(d[1] & 0xFFFF0000u));
    return r;
}

// bf16 bits -> fp16 bits, round to nearest even (exact for |v| in
// [2^-14, 65504]; larger magnitudes become infinities)
__device__ inline uint32_t bf16x2_to_f16x2_rne(uint32_t d) {
    const _Float16 lo = (_Float16)__uint_as_float(d << 16);
    const _Float16 hi = (_Float16)__uint_as_float(d & 0xFFFF0000u);
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}
__device__ inline u32x4 bf16x8_to_f16x8_rne(const u32x4& d) {
    return u32x4{bf16x2_to_f16x2_rne(d[0]), bf16x2_to_f16x2_rne(d[1]), bf16x2_to_f16x2_rne(d[2]),
                 bf16x2_to_f16x2_rne(d[3])};
}

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lds_bf16x4;

__device__ inline u32x2 lds_read_tr16(const unsigned char* p) {
    const DSA_LDS lds_bf16x4* a = (const DSA_LDS lds_bf16x4*)(p);
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((DSA_LDS lds_bf16x4*)a));
}


// max / sum over the four lanes l, l^16, l^32, l^48 (one head's column), in
// registers: v_permlane16_swap and v_permlane32_swap exchange 16-lane rows
__device__ inline float max4_rows(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum4_rows(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}


// F16: the cache's latent columns hold fp16 (see latent_to_f16_kernel) rather
// than bf16; the rope columns are bf16 either way.
template <int NH, int DL, int DR, bool F16>
struct Attend {
    using C = AttnShape<NH, DL, DR>;

    struct Smem {
        unsigned char tile[kRing][C::TILE_B];   // gathered rows, bf16 / fp16, swizzled
        int32_t sel[kMaxTopK];                  // row id per selection slot (0 where unusable)
        uint32_t valid[kMaxTopK / 32];          // selection slot t holds a usable key: bit t
        u32x4 pfrag[2][C::NHB][64];             // probabilities per head block, operand layout
        float alpha[2][C::NHB * 16];            // rescale factor per head, per tile parity
        float hsum[C::NHB * 16];                // exponent sum per head (end)
        float hmax[C::NHB * 16];                // reference maximum per head (end)
    };

    // Shared state of one block attending selected rows sel_g[t_begin ..
    // t_end) of a cache holding nkeys rows.
    struct Ctx {
        const uint16_t* kv;
        int n, ntiles;
        int w, l, g, c16;
        uint32_t lat_off[C::ILW];
        Smem* sm;
    };

    // Selection -> LDS as row ids (row 0 where a slot is unusable: past the
    // count or outside the cache) plus a validity bitmap, padded to whole
    // tiles.  Every wave calls it; ends with a barrier.
    __device__ __forceinline__ static Ctx setup(const uint16_t* kv, const int32_t* __restrict__ sel_g, int t_begin, int t_end,
                                int nkeys, Smem& sm) {
        Ctx c;
        const int tid = threadIdx.x;
        c.kv = kv;
        c.sm = &sm;
        c.w = __builtin_amdgcn_readfirstlane(tid >> 6);
        c.l = tid & 63;
        c.g = c.l >> 4;
        c.c16 = c.l & 15;
        c.n = max(t_end - t_begin, 0);
        c.ntiles = (c.n + kTK - 1) / kTK;
        const int npad = c.ntiles * kTK;
        constexpr int PER = kMaxTopK / C::NT;
        int jv[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {   // slot t = k*NT + tid: a wave covers 64 consecutive slots
            const int t = k * C::NT + tid;
            jv[k] = sel_g[t_begin + min(t, max(c.n - 1, 0))];
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int t = k * C::NT + tid;
            const bool ok = t < c.n && (unsigned)jv[k] < (unsigned)nkeys;
            if (t < npad) sm.sel[t] = ok ? jv[k] : 0;
            const uint64_t m = __ballot(ok);
            if (c.l == 0) {
                const int word = (k * C::NT + 64 * c.w) / 32;
                sm.valid[word] = (uint32_t)m;
                sm.valid[word + 1] = (uint32_t)(m >> 32);
            }
        }
        const int gw = max(c.w - C::NHB, 0);   // gather wave index (consumers)
#pragma unroll
        for (int k = 0; k < C::ILW; ++k) {
            const int i = C::ILW * gw + k;
            const int slot = i * 64 + c.l;
            const int r = slot / C::CL, pc = slot % C::CL;
            c.lat_off[k] = 16u * (uint32_t)(pc ^ (swz_lat(r) & (C::CL - 1)));
        }
        __syncthreads();
        return c;
    }

    // The gather is issued by the consumer waves only.  Issuing a tile's
    // loads occupies the wave until the CU's address unit has taken them
    // (about 64 bytes per clock for the whole CU), and the consumers have
    // the slack for it; the producers, whose scores are the critical path,
    // start their product right after the barrier.
    //
    // Cache rows one gather of a consumer wave reads: one per latent
    // instruction (wave-uniform when an instruction moves a whole row) and
    // this lane's row per rope instruction.  They are read from LDS one
    // iteration before the gather that uses them, so the gather issues
    // without waiting on LDS.
    struct Rows {
        int lat[C::ILW];
        int rope[C::IRW];
    };
    __device__ __forceinline__ static void load_rows(const Ctx& c, int it, Rows& r) {
        const Smem& sm = *c.sm;
        const int t0 = it * kTK;
        const int gw = c.w - C::NHB;
#pragma unroll
        for (int k = 0; k < C::ILW; ++k) {
            const int i = C::ILW * gw + k;
            r.lat[k] = (C::LR == 1) ? sm.sel[t0 + i] : sm.sel[t0 + (i * 64 + c.l) / C::CL];
        }
#pragma unroll
        for (int k = 0; k < C::IRW; ++k) r.rope[k] = sm.sel[t0 + ((gw + C::NG * k) * 64 + c.l) / C::CR];
    }

    // Gather tile `it` (this consumer's share) from the rows of that tile:
    // latent instruction i covers slots i*64 .. i*64+63 of the latent region
    // (row slot / CL, physical chunk slot % CL), rope instruction i likewise
    // in the rope region.  Padding chunks read chunk 0 (they meet zero query
    // columns).  With 64 chunks per latent row an instruction moves one
    // whole row: its address is wave-uniform (scalar).
    __device__ __forceinline__ static void gather(const Ctx& c, int it, const Rows& rows) {
        Smem& sm = *c.sm;
        unsigned char* buf = sm.tile[it % kRing];
        constexpr uint32_t kRowBytes = 2u * C::DQK;
        const int gw = c.w - C::NHB;
#pragma unroll
        for (int k = 0; k < C::ILW; ++k) {
            const int i = C::ILW * gw + k;
            if constexpr (C::LR == 1) {
                const int j = __builtin_amdgcn_readfirstlane(rows.lat[k]);
                gather16_to_lds(c.kv + (int64_t)j * C::DQK, c.lat_off[k], lds_addr(buf + 1024 * i));
            } else {
                gather16_to_lds(c.kv, (uint32_t)rows.lat[k] * kRowBytes + c.lat_off[k], lds_addr(buf + 1024 * i));
            }
        }
#pragma unroll
        for (int k = 0; k < C::IRW; ++k) {
            const int i = gw + C::NG * k;
            const int slot = i * 64 + c.l;
            const int r = slot / C::CR, pc = slot % C::CR;
            const int ch = pc ^ (swz_rope(r) & (C::CR - 1));
            gather16_to_lds(c.kv, (uint32_t)rows.rope[k] * kRowBytes + 2u * DL + 16u * (ch < C::CRD ? ch : 0),
                            lds_addr(buf + C::LAT_B + 1024 * i));
        }
    }

    // Consumer: wait until at most K tiles of this wave's gathers are
    // outstanding.
    template <int K>
    __device__ __forceinline__ static void wait_tiles(const Ctx& c) {
        wait_vmcnt<K * (C::ILW + C::IRW)>();
    }
    __device__ __forceinline__ static void wait_tiles_rt(const Ctx& c, int k) {   // k uniform, < kRing
        static_assert(kRing <= 5, "extend the switch");
        switch (k) {
            case 0: wait_tiles<0>(c); break;
            case 1: wait_tiles<1>(c); break;
            case 2: wait_tiles<2>(c); break;
            default: wait_tiles<3>(c); break;
        }
    }

    // Prologue shared by both roles: tiles 0 .. kRing-2 in flight, tile 0
    // landed.
    __device__ __forceinline__ static void prologue(const Ctx& c, Rows& rows) {
        if (c.w >= C::NHB) {
#pragma unroll
            for (int t = 0; t < kRing - 1; ++t) {
                if (t < c.ntiles) {
                    load_rows(c, t, rows);
                    gather(c, t, rows);
                }
            }
            if (kRing - 1 < c.ntiles) load_rows(c, kRing - 1, rows);
            if (c.ntiles > 0) wait_tiles_rt(c, min(kRing - 2, c.ntiles - 1));
        }
        __syncthreads();
    }

    // Top of iteration it, both roles: tile it+1 landed for every wave,
    // probabilities of tile it visible, tile it-1 free.  The consumers then
    // gather tile it+kRing-1 into tile it-1's buffer from inside their
    // value step (see consume).
    __device__ __forceinline__ static void step(const Ctx& c, int it) {
        // tiles it+1 .. min(it+kRing-2, ntiles-1) are in flight; keep all but it+1
        if (c.w >= C::NHB && it + 1 < c.ntiles) wait_tiles_rt(c, min(kRing - 3, c.ntiles - 2 - it));
        __syncthreads();
    }

    // Producer wave hb = w: scores and softmax of heads 16hb .. 16hb+15.
    // Leaves sm.hmax / sm.hsum per head (reference max in log2 units, sum).
    __device__ __forceinline__ static void produce(const Ctx& c, const uint16_t* __restrict__ qrow, float scale_log2) {
        Smem& sm = *c.sm;
        const int w = c.w, l = c.l, g = c.g, c16 = c.c16;
        const int head = 16 * w + c16;
        // producers are the critical path: let them issue first on their SIMD
        __builtin_amdgcn_s_setprio(2);
        const u32x4 zero = {0u, 0u, 0u, 0u};
        u32x4 qf[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const int f = 32 * ks + 8 * g;
            qf[ks] = (head < NH && f < C::DQK) ? ldg16(qrow + (int64_t)head * C::DQK + f) : zero;
        }
        if constexpr (F16) {
            // the latent part meets fp16 keys: convert (exact for |q| in
            // [2^-14, 65504], round to nearest even below)
#pragma unroll
            for (int ks = 0; ks < C::KSL; ++ks) qf[ks] = bf16x8_to_f16x8_rne(qf[ks]);
        }
        float mref = -INFINITY, lsum = 0.f;   // for head `head` (replicated over g)
        // a negative scale is folded into the query (flip the sign of every
        // 16-bit element): the scores then carry its sign and x = s * |scale|
        if (scale_log2 < 0.f) {
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) qf[ks] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        }
        const float cabs = fabsf(scale_log2);

        // Score reads: row 16mb + c16 (swizzle depends on c16 only), logical
        // chunk 4ks + g.
        const int xl = swz_lat(c16) & (C::CL - 1);
        int qlat[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) qlat[k] = c16 * C::CL * 16 + 16 * (((4 * k + g) ^ xl) & 15);
        const int xr = swz_rope(c16) & (C::CR - 1);
        int qrope[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) qrope[k] = C::LAT_B + c16 * C::CR * 16 + 16 * ((4 * k + g) ^ xr);

        auto key_frag = [&](const unsigned char* tile, int ks, u32x4 (&dst)[2]) {
            int off;
            if (ks < C::KSL) {
                off = (C::CL >= 16) ? qlat[ks & 3] + 256 * (ks >> 2)
                                    : c16 * C::CL * 16 + 16 * ((4 * ks + g) ^ xl);
            } else {
                off = qrope[(ks - C::KSL) & 1] + 128 * ((ks - C::KSL) >> 1);
            }
            const int rs = (ks < C::KSL) ? C::CL * 16 : C::CR * 16;   // bytes per row
            dst[0] = *reinterpret_cast<const u32x4*>(tile + off);
            dst[1] = *reinterpret_cast<const u32x4*>(tile + off + 16 * rs);
        };
        auto score = [&](int it) {
            const unsigned char* tile = sm.tile[it % kRing];
            // validity of the tile's 32 keys: bit k is key t0 + k
            const uint32_t vmask = sm.valid[it];
            f32x4 s[2] = {};
            constexpr int KR = kKeyAhead + 1;
            u32x4 ka[KR][2];   // key fragments, kKeyAhead k-steps ahead of their MFMAs
#pragma unroll
            for (int ks = 0; ks < kKeyAhead && ks < C::KS; ++ks) key_frag(tile, ks, ka[ks]);
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                if (ks + kKeyAhead < C::KS) key_frag(tile, ks + kKeyAhead, ka[(ks + kKeyAhead) % KR]);
                asm volatile("" ::: "memory");
                if (F16 && ks < C::KSL) {
                    s[0] = mfma16_f16(ka[ks % KR][0], qf[ks], s[0]);
                    s[1] = mfma16_f16(ka[ks % KR][1], qf[ks], s[1]);
                } else {
                    s[0] = mfma16_bf16(ka[ks % KR][0], qf[ks], s[0]);
                    s[1] = mfma16_bf16(ka[ks % KR][1], qf[ks], s[1]);
                }
            }
            // x = s * scale (log2 units) = sv * cabs; unusable keys -> -inf
            float sv[8];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int i = 0; i < 4; ++i) sv[4 * mb + i] = s[mb][i];
            if (vmask != 0xFFFFFFFFu) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (!((vmask >> (16 * mb + 4 * g + i)) & 1u)) sv[4 * mb + i] = -INFINITY;
            }
            // The exponentials go against the current reference while the
            // tile maximum is formed alongside.  The lazy reference moves
            // only when a score clears it by kLazy (always on the first tile
            // with a usable key; the output is then still zero and needs no
            // rescale), and only then are the exponentials redone, so the
            // maximum stays off the critical path.  Arguments are <= kLazy;
            // v_exp_f32 returns 0 for -inf.
            float mbase = (mref == -INFINITY) ? 0.f : mref;
            float p[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], cabs, -mbase));
            float mx = sv[0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
            mx = max4_rows(mx) * cabs;
            const bool up = mx > mref + kLazy;
            float alpha = 1.f;
            if (__ballot(up)) {   // wave-uniform and rare
                alpha = (up && mref != -INFINITY) ? __builtin_amdgcn_exp2f(mref - mx) : 1.f;
                mref = up ? mx : mref;
                mbase = (mref == -INFINITY) ? 0.f : mref;
#pragma unroll
                for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], cabs, -mbase));
            }
            u32x4 pb;
            pb[0] = pack_f16(p[0], p[1]);
            pb[1] = pack_f16(p[2], p[3]);
            pb[2] = pack_f16(p[4], p[5]);
            pb[3] = pack_f16(p[6], p[7]);
            sm.pfrag[it & 1][w][l] = pb;
            sm.alpha[it & 1][head] = alpha;   // the four lanes of a head store the same value
            float ps = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ps += p[i];
            lsum = lsum * alpha + ps;
        };

        Rows rows;
        prologue(c, rows);
        if (c.ntiles > 0) score(0);
        for (int it = 0; it < c.ntiles; ++it) {
            step(c, it);
            if (it + 1 < c.ntiles) score(it + 1);
        }
        lsum = sum4_rows(lsum);
        if (g == 0) { sm.hsum[head] = lsum; sm.hmax[head] = mref; }
        __syncthreads();
    }

    // Consumer wave cw = w - NHB: accumulates o[f][hb], the unnormalised
    // output of head 16hb + (lane & 15) and features
    // 16(FBW cw + f) + 4(lane >> 4) + i.
    __device__ __forceinline__ static void consume(const Ctx& c, f32x4 (&o)[C::FBW][C::NHB]) {
        Smem& sm = *c.sm;
        const int l = c.l, g = c.g, c16 = c.c16;
        const int cw = c.w - C::NHB;
#pragma unroll
        for (int f = 0; f < C::FBW; ++f)
#pragma unroll
            for (int hb = 0; hb < C::NHB; ++hb) o[f][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // transposed reads: rows 16h + 4g + (c16 >> 2), features
        // 16fb + 4(c16 & 3): logical chunk 2fb + ((c16 >> 1) & 1), half c16 & 1
        const int trow = 4 * g + (c16 >> 2);
        const int vx = (swz_lat(trow) & (C::CL - 1)) ^ ((c16 >> 1) & 1);
        const int vrow = trow * C::CL * 16 + 8 * (c16 & 1);

        Rows rows;
        auto values = [&](int it) {
            // The row ids (read an iteration ago) are taken before this
            // tile's LDS reads go out; otherwise the first gather
            // instruction waits for those reads too.
#pragma unroll
            for (int k = 0; k < C::ILW; ++k) asm volatile("" :: "v"(rows.lat[k]));
#pragma unroll
            for (int k = 0; k < C::IRW; ++k) asm volatile("" :: "v"(rows.rope[k]));
            u32x4 pf[C::NHB];
            float al[C::NHB];
            bool moved = false;
#pragma unroll
            for (int hb = 0; hb < C::NHB; ++hb) {
                pf[hb] = sm.pfrag[it & 1][hb][l];
                al[hb] = sm.alpha[it & 1][16 * hb + c16];
                moved |= al[hb] != 1.f;
            }
            const unsigned char* tile = sm.tile[it % kRing];
            // Every value fragment of the tile is read up front and pinned
            // there: left alone, the scheduler sinks each transposing read
            // next to its MFMAs (a compiler memory fence does not hold these
            // read intrinsics), and every MFMA waits out an LDS latency.
            u32x2 vr[C::FBW][2];
#pragma unroll
            for (int f = 0; f < C::FBW; ++f) {
                const int fb = C::FBW * cw + f;
                // logical chunk 2fb + tb, swizzled in its aligned group of 16
                const int off = vrow + 16 * (((2 * fb) & ~15) + (((2 * fb) & 15) ^ vx));
                vr[f][0] = lds_read_tr16(tile + off);
                vr[f][1] = lds_read_tr16(tile + off + 16 * C::CL * 16);
            }
            __builtin_amdgcn_sched_barrier(0);
            // The next gather goes out behind this wave's LDS reads, never
            // ahead of them: an LDS read issued after LDS-DMA loads waits
            // until the address unit has taken those loads.  Its rows were
            // read in the previous iteration.
            if (it + kRing - 1 < c.ntiles) gather(c, it + kRing - 1, rows);
            __builtin_amdgcn_sched_barrier(0);
            if (__ballot(moved)) {   // wave-uniform and rare
#pragma unroll
                for (int f = 0; f < C::FBW; ++f)
#pragma unroll
                    for (int hb = 0; hb < C::NHB; ++hb) o[f][hb] *= al[hb];
            }
#pragma unroll
            for (int f = 0; f < C::FBW; ++f) {
                u32x2 v0 = vr[f][0], v1 = vr[f][1];
                if constexpr (!F16) {
                    v0 = bf16x4_to_f16x4(v0);
                    v1 = bf16x4_to_f16x4(v1);
                }
                const u32x4 av = {v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
                for (int hb = 0; hb < C::NHB; ++hb) o[f][hb] = mfma16_f16(av, pf[hb], o[f][hb]);
            }
            // rows of the following gather, after the MFMAs have issued
            __builtin_amdgcn_sched_barrier(0);
            if (it + kRing < c.ntiles) load_rows(c, it + kRing, rows);
        };

        prologue(c, rows);
        for (int it = 0; it < c.ntiles; ++it) {
            step(c, it);
            values(it);
        }
        __syncthreads();
    }
};

template <int NH, int DL, int DR, bool F16>
__global__ __launch_bounds__((AttnShape<NH, DL, DR>::NT)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_kernel(AttnArgs a) {
    using C = AttnShape<NH, DL, DR>;
    using A = Attend<NH, DL, DR, F16>;
    __shared__ __attribute__((aligned(16))) typename A::Smem sm;
    const int row = blockIdx.x;
    const int cnt = min(max(a.count[row], 0), a.top_k);
    const auto c = A::setup(a.kv, a.idx + (int64_t)row * a.top_k, 0, cnt, a.N, sm);
    if (c.w < C::NHB) {
        A::produce(c, a.q + (int64_t)row * NH * C::DQK, a.scale_log2);
        if (a.lse && c.w == 0 && c.l < 16) {
            for (int h = c.l; h < NH; h += 16) {
                const float ls = sm.hsum[h];
                a.lse[(int64_t)row * NH + h] = ls > 0.f ? (sm.hmax[h] + log2f(ls)) * 0.69314718055994531f : -INFINITY;
            }
        }
    } else {
        f32x4 o[C::FBW][C::NHB];
        A::consume(c, o);
        const int cw = c.w - C::NHB;
#pragma unroll
        for (int hb = 0; hb < C::NHB; ++hb) {
            const int head = 16 * hb + c.c16;
            if (head >= NH) continue;
            const float ls = sm.hsum[head];
            const float inv = ls > 0.f ? 1.f / ls : 0.f;
            float* orow = a.out + ((int64_t)row * NH + head) * DL;
#pragma unroll
            for (int f = 0; f < C::FBW; ++f)
                *reinterpret_cast<f32x4*>(orow + 16 * (C::FBW * cw + f) + 4 * c.g) = o[f][hb] * inv;
        }
    }
}

// The decode selection of one attention block: slots [t_begin, t_end) of
// sequence b's ascending selection go to dsel (LDS) and out to idx.
struct DecSelSmem {
    int32_t sure[kMaxTopK];   // keys above the boundary bin, ascending
    int32_t ck[kDecCap];      // candidates (boundary-bin keys), ascending
    float cv[kDecCap];        // and their scores
    int32_t kept[kDecCap];    // the kept candidates, ascending
    int32_t dsel[kMaxTopK];   // this block's slots
    int wcnt[16];
};

// Returns where the block's selection slots are (t_begin shifted to 0 when
// they were built in LDS).  A sequence of at most top_k keys selects every
// key; a sequence the top-k fallback selected is read from idx; otherwise
// the candidates are ranked (higher score, then lower key: a strict order),
// the best top_k - above are kept, and each slot of the block takes its
// element of the merge of the sure and kept lists.  Every thread calls it;
// the slots it built in LDS are complete (behind a barrier) when it returns.
template <int NT>
__device__ __forceinline__ const int32_t* decode_selection(const AttnSplitArgs& a, const SeqMeta& m, int b,
                                                           bool first, int& t_begin, int& t_end,
                                                           DecSelSmem& ds) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ctx = m.ctx[b], top_k = a.top_k;
    int32_t* idx_b = a.idx + (int64_t)b * top_k;
    const int n = t_end - t_begin;
    if (ctx <= top_k) {
        for (int t = tid; t < n; t += NT) {
            ds.dsel[t] = t_begin + t;
            idx_b[t_begin + t] = t_begin + t;
        }
        if (first) {
            for (int t = ctx + tid; t < top_k; t += NT) idx_b[t] = -1;
            if (tid == 0) a.count[b] = ctx;
        }
        __syncthreads();
        t_end -= t_begin;
        t_begin = 0;
        return ds.dsel;
    }
    // one round of loads: the sequence's counts and both lists at their full
    // capacity (entries past the counts are ignored)
    constexpr int SP = kMaxTopK / NT, CP = (kDecCap + NT - 1) / NT;
    int32_t sv[SP];
    DecCand cv[CP];
    const int32_t* sure_g = a.dec.sure + (int64_t)b * top_k;
    const DecCand* cand_g = a.dec.cand + (int64_t)b * kDecCap;
#pragma unroll
    for (int k = 0; k < SP; ++k) sv[k] = k * NT + tid < top_k ? sure_g[k * NT + tid] : 0;
#pragma unroll
    for (int k = 0; k < CP; ++k) cv[k] = k * NT + tid < kDecCap ? cand_g[k * NT + tid] : DecCand{0, 0.f};
    const DecSeqInfo info = a.dec.info[b];
    if (info.degenerate || info.fallback) return idx_b;
    const int above = info.above, inbin = info.inbin, krem = top_k - above;   // 1 <= krem <= inbin
#pragma unroll
    for (int k = 0; k < SP; ++k)
        if (k * NT + tid < above) ds.sure[k * NT + tid] = sv[k];
#pragma unroll
    for (int k = 0; k < CP; ++k)
        if (k * NT + tid < inbin) {
            ds.ck[k * NT + tid] = cv[k].key;
            ds.cv[k * NT + tid] = cv[k].score;
        }
    __syncthreads();
    // kept candidates, in list (= key) order: each candidate is ranked by P
    // consecutive lanes (P = 16 for up to NT / 16 candidates)
    int lg = 0;
    while (lg < 4 && (inbin << (lg + 1)) <= NT) ++lg;
    const int P = 1 << lg;
    int base = 0;
    for (int c0 = 0; c0 < inbin; c0 += NT >> lg) {
        const int ci = c0 + (tid >> lg), part = tid & (P - 1);
        int r = 0;
        if (ci < inbin) {
            const float v = ds.cv[ci];
            const int32_t kc = ds.ck[ci];
            for (int i = part; i < inbin; i += P) {
                const float x = ds.cv[i];
                r += (x > v || (x == v && ds.ck[i] < kc)) ? 1 : 0;
            }
        }
        r = group_sum(r, P);
        const bool keep = ci < inbin && part == 0 && r < krem;
        const uint64_t mk = __ballot(keep);
        if (lane == 0) ds.wcnt[wave] = __popcll(mk);
        __syncthreads();
        int off = base, tot = 0;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) {
            const int x = ds.wcnt[w];
            off += w < wave ? x : 0;
            tot += x;
        }
        if (keep) ds.kept[off + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0))] = ds.ck[ci];
        base += tot;
        __syncthreads();
    }
    // slot p of the merged list (merge path): i = sure keys among the first
    // p, found by bisection over the at most krem + 1 possible splits (sure
    // and kept keys are distinct), then the smaller of sure[i] and kept[p - i]
    for (int t = tid; t < n; t += NT) {
        const int p = t_begin + t;
        int lo = max(0, p - krem), hi = min(p, above);
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (ds.sure[mid] < ds.kept[p - 1 - mid]) lo = mid + 1;
            else hi = mid;
        }
        const int j = p - lo;
        ds.dsel[t] = (j >= krem || (lo < above && ds.sure[lo] < ds.kept[j])) ? ds.sure[lo] : ds.kept[j];
    }
    __syncthreads();
    for (int t = tid; t < n; t += NT) idx_b[t_begin + t] = ds.dsel[t];
    if (first && tid == 0) a.count[b] = top_k;
    t_end -= t_begin;
    t_begin = 0;
    return ds.dsel;
}

template <int NH, int DL, int DR>
__global__ __launch_bounds__((AttnShape<NH, DL, DR>::NT)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_split_kernel(AttnSplitArgs a, SeqMeta m) {
    using C = AttnShape<NH, DL, DR>;
    using A = Attend<NH, DL, DR, false>;
    __shared__ __attribute__((aligned(16))) typename A::Smem sm;
    __shared__ DecSelSmem ds;
    const int item = blockIdx.x;
    const int b = seq_of_block(m, item);
    const int ctx = m.ctx[b];
    const int cnt = min(ctx, a.top_k);
    int t_begin = (item - m.blk0[b]) * a.chunk;
    int t_end = min(t_begin + a.chunk, cnt);
    const int32_t* sel = decode_selection<C::NT>(a, m, b, item == m.blk0[b], t_begin, t_end, ds);
    const auto c = A::setup(a.kv + m.key_off[b] * C::DQK, sel, t_begin, t_end, ctx, sm);
    if (c.w < C::NHB) {
        A::produce(c, a.q + (int64_t)b * NH * C::DQK, a.scale_log2);
        if (c.w == 0 && c.l < 16) {
            for (int h = c.l; h < NH; h += 16) {
                a.part_ml[((int64_t)item * NH + h) * 2 + 0] = sm.hmax[h];
                a.part_ml[((int64_t)item * NH + h) * 2 + 1] = sm.hsum[h];
            }
        }
    } else {
        f32x4 o[C::FBW][C::NHB];
        A::consume(c, o);
        const int cw = c.w - C::NHB;
#pragma unroll
        for (int hb = 0; hb < C::NHB; ++hb) {
            const int head = 16 * hb + c.c16;
            if (head >= NH) continue;
            float* orow = a.part_o + ((int64_t)item * NH + head) * DL;
#pragma unroll
            for (int f = 0; f < C::FBW; ++f)
                // streamed past the L2 (the combine reads them on other XCDs):
                // less to write back when the launch ends
                __builtin_nontemporal_store(o[f][hb], reinterpret_cast<f32x4*>(orow + 16 * (C::FBW * cw + f) + 4 * c.g));
        }
    }
}

// kv16 = kv with the Dl latent columns of every row converted bf16 -> fp16
// (round to nearest even; exact for |v| in [2^-14, 65504]) and the rope
// columns copied.  One thread per 16-byte chunk.
template <int DL, int DR>
__global__ __launch_bounds__(256) void latent_to_f16_kernel(const uint16_t* __restrict__ kv,
                                                            uint16_t* __restrict__ kv16, int64_t nchunks) {
    constexpr int CPR = (DL + DR) / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= nchunks) return;
    const int ch = (int)(gid % CPR);
    u32x4 v = ldg16(kv + gid * 8);
    if (ch < DL / 8) v = bf16x8_to_f16x8_rne(v);
    *reinterpret_cast<u32x4*>(kv16 + gid * 8) = v;
}

// out[b,h,:] = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c over the chunks
// c of sequence b.  Wave 0 turns the chunks' (m, l) into one weight per chunk
// (lane c holds chunk c; M and the denominator are wave reductions); then
// every thread owns four features and issues the loads of all chunks back to
// back.  Chunks without a usable key have m = -inf and weight 0 (their
// partial output is zero).
template <int NH, int DL>
__global__ __launch_bounds__(128) void combine_kernel(AttnSplitArgs a, SeqMeta m) {
    constexpr int kMaxChunks = kMaxTopK / kTK;   // chunks hold at least one tile
    static_assert(kMaxChunks <= 64, "one lane per chunk");
    __shared__ float wgt[kMaxChunks];
    const int b = blockIdx.x / NH, h = blockIdx.x % NH;
    const int it0 = m.blk0[b];
    const int n = min(m.blk0[b + 1] - it0, kMaxChunks);
    const int tid = threadIdx.x;
    if (tid < 64) {
        float mi = -INFINITY, li = 0.f;
        if (tid < n) {
            mi = a.part_ml[((int64_t)(it0 + tid) * NH + h) * 2];
            li = a.part_ml[((int64_t)(it0 + tid) * NH + h) * 2 + 1];
        }
        float M = mi;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        const float e = (mi == -INFINITY) ? 0.f : exp2f(mi - M);
        float den = e * li;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
        const float inv = den > 0.f ? 1.f / den : 0.f;
        if (tid < kMaxChunks) wgt[tid] = tid < n ? e * inv : 0.f;
    }
    __syncthreads();
    for (int f = 4 * tid; f < DL; f += 4 * 128) {
        const float* po = a.part_o + ((int64_t)it0 * NH + h) * DL + f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        int c = 0;
        for (; c + 8 <= n; c += 8) {
            f32x4 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const f32x4*>(po + (int64_t)(c + k) * NH * DL);
#pragma unroll
            for (int k = 0; k < 8; ++k) acc += wgt[c + k] * v[k];
        }
        for (; c < n; ++c) acc += wgt[c] * *reinterpret_cast<const f32x4*>(po + (int64_t)c * NH * DL);
        *reinterpret_cast<f32x4*>(a.out + ((int64_t)b * NH + h) * DL + f) = acc;
    }
}

}  // namespace

hipError_t launch_attention(int shape_id, const AttnArgs& a, bool kv_f16, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    const dim3 grid(a.rows);
    if (shape_id == 0) {
        if (kv_f16) hipLaunchKernelGGL((attention_kernel<64, 512, 64, true>), grid, dim3(AttnShape<64, 512, 64>::NT), 0, s, a);
        else hipLaunchKernelGGL((attention_kernel<64, 512, 64, false>), grid, dim3(AttnShape<64, 512, 64>::NT), 0, s, a);
    } else {
        if (kv_f16) hipLaunchKernelGGL((attention_kernel<4, 64, 16, true>), grid, dim3(AttnShape<4, 64, 16>::NT), 0, s, a);
        else hipLaunchKernelGGL((attention_kernel<4, 64, 16, false>), grid, dim3(AttnShape<4, 64, 16>::NT), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_latent_to_f16(int shape_id, const uint16_t* kv, uint16_t* kv16, int64_t rows, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const int cpr = shape_id == 0 ? (512 + 64) / 8 : (64 + 16) / 8;
    const int64_t nchunks = rows * cpr;
    const dim3 grid((unsigned)((nchunks + 255) / 256));
    if (shape_id == 0) hipLaunchKernelGGL((latent_to_f16_kernel<512, 64>), grid, dim3(256), 0, s, kv, kv16, nchunks);
    else hipLaunchKernelGGL((latent_to_f16_kernel<64, 16>), grid, dim3(256), 0, s, kv, kv16, nchunks);
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
