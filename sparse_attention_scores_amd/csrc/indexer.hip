// indexer.hip - DSA indexer scores on gfx950 MFMA.
//
// exo PR #2539 (glm_moe_dsa attention speed-ups), Prefill section, float32
// indexer item: a key's score for a query is the sum over the indexer heads
// of the head weight times relu(q.k), accumulated in float32 in one pass with
// the causal mask applied.  One Di-wide indexer key per token is shared by
// all heads.
//
// Design: the product for one query is a [heads x Di] x [Di x keys] GEMM, so
// the 32 indexer heads are the 32 rows of a v_mfma_f32_32x32x16_bf16 tile and
// 32 keys its columns.  In the 32x32 accumulator layout a lane holds 16 of
// the 32 heads of one key, so the weighted relu sum over heads is 16 FMAs in
// the lane plus one exchange with lane l^32 (v_permlane32_swap), which also
// packs two results per lane.  bf16 products of integers are exact and the
// fp32 sum is exact while it stays below 2^24.
//
// Prefill: a block holds 16 queries (2 per wave, their Q fragments and
// weights stay in VGPRs) and streams a key tile through LDS in 128-key
// double-buffered stages, so each key row is read from L2 once per 16
// queries.  The tile is all keys when there are enough query blocks to fill
// the chip (each query block's fragments are then loaded once), else the
// keys are split so that the grid covers every compute unit.  Tiles past the
// block's last causal key are not computed.
// Decode: one query per sequence, so no reuse across queries: each wave
// copies 64 key rows to LDS with whole-row loads and scores them from there
// against the block's one LDS copy of the query (the step is HBM bound).
#include "dsa_kernels.h"

#include <math.h>

namespace dsa {
namespace {

template <int HI, int DI>
struct IdxShape {
    static_assert(HI <= 32 && HI % 4 == 0, "indexer heads must fit one 32-row MFMA tile");
    static_assert(DI % 16 == 0, "indexer width must be a multiple of the MFMA K step");
    static constexpr int KS = DI / 16;        // 32x32x16 K steps
    static constexpr int ROWB = DI * 2 + 16;  // LDS bytes per key row, padded against bank conflicts
    static constexpr int CPR = DI / 8;        // 16-byte pieces per key row
};

constexpr int kIdxWaves = 8;
constexpr int kIdxThreads = kIdxWaves * 64;
constexpr int kIdxQPB = kIdxWaves * 2;   // queries per block
constexpr int kIdxSub = 128;             // keys per LDS stage
constexpr int kIdxChunks = kIdxSub / 32; // 32-key MFMA chunks per stage
constexpr int kIdxCUs = 256;              // compute units the grid should cover

constexpr int kIdxdWaves = 4;
constexpr int kIdxdSlab = 64;                                // keys per LDS slab
constexpr int kIdxdSlabs = 2;                                // slabs per wave, one after the other
constexpr int kIdxdKeysPerWave = kIdxdSlab * kIdxdSlabs;
constexpr int kIdxdKeysPerBlock = kIdxdWaves * kIdxdKeysPerWave;

// Head held by accumulator register r of lane-half `half` in the 32x32 layout.
__device__ inline int acc_head(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// The weights of the 16 heads this lane's accumulator holds for query q
// (heads past HI weigh zero).
template <int HI>
__device__ __forceinline__ void load_weights(const float* w, int64_t q, int half, float (&wr)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int h = acc_head(r, half);
        const float v = w[q * HI + (h < HI ? h : HI - 1)];
        wr[r] = h < HI ? v : 0.f;
    }
}

// Query q's MFMA A fragments (rows = heads) and its head weights.  Loads are
// unconditional (q must be a valid row); rows past HI read as zero.
template <int HI, int DI>
__device__ __forceinline__ void load_query(const uint16_t* qI, const float* w, int64_t q, int col,
                                           int half, u32x4 (&qf)[IdxShape<HI, DI>::KS],
                                           float (&wr)[16]) {
    using C = IdxShape<HI, DI>;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const int hc = col < HI ? col : HI - 1;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        const u32x4 v = ldg16(qI + (q * HI + hc) * DI + ks * 16 + half * 8);
        qf[ks] = col < HI ? v : zero;
    }
    load_weights<HI>(w, q, half, wr);
}

// A wave-uniform address held in SGPRs.  readfirstlane returns int, so each
// half is widened through uint32_t (the low half must not be sign-extended).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return (const void*)(((uint64_t)hi << 32) | lo);
}

// relu as one integer max: a float's bit pattern read as int32 is negative
// exactly when its sign bit is set, so max(bits, 0) maps every negative
// value (and -0) to +0 and keeps the rest.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// sum over this lane's 16 heads of w * relu(score)
__device__ __forceinline__ float weighted_relu(const f32x16& acc, const float (&wr)[16]) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s = fmaf(wr[r], relu(acc[r]), s);
    return s;
}

// lanes 0-31 get x summed over both halves, lanes 32-63 get y summed likewise
__device__ __forceinline__ float combine_halves(float x, float y) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Prefill: block = 16 queries (two per wave: lanes 0-31 report the first,
// lanes 32-63 the second) x a key tile, streamed through LDS in 128-key
// stages (double-buffered, filled by direct global-to-LDS loads).  The loop
// is software-pipelined by one 32-key chunk: the MFMAs of chunk g are
// interleaved with the relu-weighted head sum of chunk g-1, so the vector
// ALU work runs under the matrix unit.  Results are stored once per stage,
// right after the wait for the stage's loads (which also covers stores), so
// the stores have a whole stage to drain before the next wait.
template <int HI, int DI>
__global__ __launch_bounds__(kIdxThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void indexer_prefill_kernel(IndexerArgs a) {
    using C = IdxShape<HI, DI>;
    constexpr int STAGE_B = kIdxSub * C::ROWB;            // LDS bytes per stage
    static_assert(STAGE_B % 1024 == 0, "a stage must be whole 64-slot runs");
    constexpr int NRUN = STAGE_B / 1024;                  // 64-slot DMA runs per stage
    constexpr int RUNS = (NRUN + kIdxWaves - 1) / kIdxWaves;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2][STAGE_B];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int half = lane >> 5, col = lane & 31;
    const int q_base = blockIdx.y * kIdxQPB;
    const int q_last = min(q_base + kIdxQPB, a.rows) - 1;
    const int64_t p_last = a.pos0 + q_last;
    const int key_beg = blockIdx.x * a.key_tile;
    const int key_tile_end = min(key_beg + a.key_tile, a.N);
    const int kend = (int)min<int64_t>((int64_t)key_tile_end, p_last + 1);

    if (a.write_masked) {   // keys every query of the block masks
        const int m0 = max(kend, key_beg);
        const int width = key_tile_end - m0;
        if (width > 0) {
            const int n = (q_last - q_base + 1) * width;
            for (int e = tid; e < n; e += kIdxThreads)
                a.S[(int64_t)(q_base + e / width) * a.ldS + m0 + e % width] = -INFINITY;
        }
    }
    if (kend <= key_beg) return;

    // this lane's query (waves past the last row compute a copy and store nothing)
    const int qa = min(q_base + 2 * wave, q_last), qb = min(q_base + 2 * wave + 1, q_last);
    const int myq = q_base + 2 * wave + half;
    const bool vq = myq <= q_last;
    const int64_t myp = a.pos0 + myq;
    float* srow = a.S + (int64_t)myq * a.ldS;

    u32x4 qfa[C::KS], qfb[C::KS];
    float wa[16], wb[16];
    load_query<HI, DI>(a.qI, a.w, qa, col, half, qfa, wa);
    load_query<HI, DI>(a.qI, a.w, qb, col, half, qfb, wb);

    // A stage is kIdxSub padded rows of ROWB bytes, i.e. SLOTS 16-byte slots
    // in LDS order; row r's slot p < CPR holds piece p of key row
    // (stage base + r), its padding slot a copy of piece 0.  Wave w fills
    // the 64-slot runs w, w + 8, ... by DMA, each lane one slot.  Rows past
    // the last key read the last key (never stored).
    const uint32_t lds0 = lds_addr(&lds[0][0]);
    const uint32_t kI_bytes_max = (uint32_t)(a.N - 1) * (uint32_t)(DI * 2);
    auto dma = [&](int s, int buf) {
        const int row0 = key_beg + s * kIdxSub;
#pragma unroll
        for (int c = 0; c < RUNS; ++c) {
            const int run = wave + c * kIdxWaves;
            if (RUNS * kIdxWaves == NRUN || run < NRUN) {
                const int slot = run * 64 + lane;
                const int r = slot / (C::CPR + 1), p = slot - r * (C::CPR + 1);
                const uint32_t off = min((uint32_t)(row0 + r) * (uint32_t)(DI * 2), kI_bytes_max) +
                                     (uint32_t)(p < C::CPR ? p : 0) * 16u;
                gather16_to_lds(a.kI, off, lds0 + buf * STAGE_B + run * 1024);
            }
        }
    };
    // store the head sum of flat chunk g (lanes: this lane's query, key g*32+col)
    auto put = [&](int g, float v) {
        const int key = key_beg + g * 32 + col;
        if (g >= 0 && vq && key < kend) {
            if (key <= myp) srow[key] = v;
            else if (a.write_masked) srow[key] = -INFINITY;
        }
    };

    const int nsub = (kend - key_beg + kIdxSub - 1) / kIdxSub;
    dma(0, 0);
    if (nsub > 1) dma(1, 1);
    wait_vmcnt<0>();
    __syncthreads();

    f32x16 pa = {}, pb = {};   // accumulators of the previous chunk
    constexpr int NSTEP = kIdxChunks * C::KS;   // (chunk, k-step) pairs per stage
    for (int s = 0; s < nsub; ++s) {
        const unsigned char* buf = lds[s & 1] + col * C::ROWB + half * 16;
        auto bread = [&](int i) {
            return *reinterpret_cast<const u32x4*>(buf + 32 * (i / C::KS) * C::ROWB + (i % C::KS) * 32);
        };
        float res[kIdxChunks];
        u32x4 br[3];   // key fragments, read two k-steps ahead
        br[0] = bread(0);
        br[1] = bread(1);
        f32x16 ca = {}, cb = {};
#pragma unroll
        for (int i = 0; i < NSTEP; ++i) {
            const int ks = i % C::KS;
            if (i + 2 < NSTEP) br[(i + 2) % 3] = bread(i + 2);
            if (ks == 0) ca = cb = f32x16{};
            ca = mfma32_bf16(qfa[ks], br[i % 3], ca);
            cb = mfma32_bf16(qfb[ks], br[i % 3], cb);
            if (ks == C::KS - 1) {
                res[i / C::KS] = combine_halves(weighted_relu(pa, wa), weighted_relu(pb, wb));
                pa = ca;
                pb = cb;
            }
        }
        // stage s+1 has landed and every wave is done with stage s, whose
        // buffer then takes stage s+2; the stores drain during stage s+1
        wait_vmcnt<0>();
        __syncthreads();
        if (s + 2 < nsub) dma(s + 2, s & 1);
#pragma unroll
        for (int t = 0; t < kIdxChunks; ++t) put(s * kIdxChunks + t - 1, res[t]);
    }
    put(nsub * kIdxChunks - 1, combine_halves(weighted_relu(pa, wa), weighted_relu(pb, wb)));
}

// Decode: each wave scores 64 consecutive keys of one sequence.  A load of
// MFMA operands straight from memory touches 32 rows at 32 bytes each, which
// costs far more memory-pipeline work per byte than whole rows, so rows go to
// LDS first with direct global-to-LDS loads (each instruction moves 64/CPR
// whole rows) and the operands are read back from there: each wave copies
// its 64 key rows to a slab of its own, and the block's waves copy the
// sequence's query (HI rows) once for all of them.  Row r's 16-byte piece c
// sits at position c ^ (r mod CPR) of the row, so the 16 lanes of one
// ds_read_b128 cycle (16 rows, one piece each) hit 16 different bank groups.
// Key rows past the context read the last key (their scores are not stored).
template <int HI, int DI>
__global__ __launch_bounds__(kIdxdWaves * 64)
void indexer_decode_kernel(const uint16_t* __restrict__ qI, const uint16_t* __restrict__ kI,
                           const float* __restrict__ w, float* __restrict__ S, SeqMeta m) {
    using C = IdxShape<HI, DI>;
    static_assert(kIdxdSlab == 64, "a slab is two 32-key MFMA tiles");
    constexpr int SLOTS = kIdxdSlab * C::CPR;   // 16-byte slots of a key slab
    constexpr int QS = HI * C::CPR;             // 16-byte slots of the query
    constexpr int QRUNS = (QS + 63) / 64;       // 64-slot copies of the query
    __shared__ u32x4 lds[kIdxdWaves][SLOTS];
    __shared__ u32x4 ldq[QRUNS * 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, col = lane & 31;
    const int b = seq_of_block(m, blockIdx.x);
    const int ctx = m.ctx[b];
    const int kw = (blockIdx.x - m.blk0[b]) * kIdxdKeysPerBlock + wave * kIdxdKeysPerWave;
    const uint32_t slab = lds_addr(&lds[wave][0]);
    // whole key rows of the slab at key kb to this wave's LDS slab (rows past
    // the sequence repeat its last key, never stored); piece p of row r sits
    // at slot p ^ (r mod CPR)
    auto copy_slab = [&](int kb) {
        const void* kbase = uniform_ptr(kI + (m.key_off[b] + kb) * DI);
        const int last = min(kIdxdSlab - 1, ctx - 1 - kb);
#pragma unroll
        for (int i = 0; i < C::CPR; ++i) {
            const int slot = i * 64 + lane, r = slot / C::CPR, p = slot % C::CPR;
            const int piece = p ^ (r % C::CPR);
            gather16_to_lds(kbase, (uint32_t)(min(r, last) * DI * 2 + piece * 16), slab + i * 1024);
        }
    };
    const bool live = kw < ctx;   // wave-uniform; idle waves still help with the query
    if (live) copy_slab(kw);
    {
        const void* qbase = uniform_ptr(qI + (int64_t)b * HI * DI);
        for (int i = wave; i < QRUNS; i += kIdxdWaves) {
            // lanes past the query's slots copy its last slot (never read)
            const int slot = min(i * 64 + lane, QS - 1), r = slot / C::CPR, p = slot % C::CPR;
            gather16_to_lds(qbase, (uint32_t)(r * DI * 2 + (p ^ (r % C::CPR)) * 16), lds_addr(&ldq[i * 64]));
        }
    }
    // the sequence's head weights: uniform addresses (scalar loads), the
    // lane's 16 picked by its half
    float wr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int h0 = acc_head(r, 0), h1 = acc_head(r, 1);
        const float w0 = h0 < HI ? w[b * HI + h0] : 0.f, w1 = h1 < HI ? w[b * HI + h1] : 0.f;
        wr[r] = half ? w1 : w0;
    }
    wait_vmcnt<0>();
    __syncthreads();
    if (!live) return;

    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 qf[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        const int pos = (ks * 2 + half) ^ (col % C::CPR);
        qf[ks] = col < HI ? ldq[col * C::CPR + pos] : zero;
    }
    for (int j = 0; j < kIdxdSlabs; ++j) {
        const int kb = kw + j * kIdxdSlab;
        u32x4 b0[C::KS], b1[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const int pos = (ks * 2 + half) ^ (col % C::CPR);   // rows col and col + 32 share the swizzle
            b0[ks] = lds[wave][col * C::CPR + pos];
            b1[ks] = lds[wave][(col + 32) * C::CPR + pos];
        }
        // the next slab reuses this one's LDS once its reads have returned;
        // its copy then runs under this slab's MFMAs and store
        const bool next = j + 1 < kIdxdSlabs && kb + kIdxdSlab < ctx;
        if (next) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            copy_slab(kb + kIdxdSlab);
        }
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            acc0 = mfma32_bf16(qf[ks], b0[ks], acc0);
            acc1 = mfma32_bf16(qf[ks], b1[ks], acc1);
        }
        const float tot = combine_halves(weighted_relu(acc0, wr), weighted_relu(acc1, wr));
        const int key = kb + 32 * half + col;
        if (key < ctx) S[m.s_off[b] + key] = tot;   // the query sits at ctx-1: every cached key is visible
        if (!next) break;
        // the copy's loads precede this store: all but the newest access done
        wait_vmcnt<1>();
    }
}

}  // namespace

int indexer_decode_keys_per_block() { return kIdxdKeysPerBlock; }

hipError_t launch_indexer_prefill(int shape_id, const IndexerArgs& a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    // key rows are addressed with 32-bit byte offsets (one stage past N included)
    const int64_t row_bytes = shape_id == 0 ? 256 : 64;
    if (((int64_t)a.N + kIdxSub) * row_bytes > 0xFFFFFFFFll) return hipErrorInvalidValue;
    const int qblocks = (a.rows + kIdxQPB - 1) / kIdxQPB;
    const int ntiles = max(1, min((kIdxCUs + qblocks - 1) / qblocks, (a.N + kIdxSub - 1) / kIdxSub));
    IndexerArgs b = a;
    b.key_tile = ((a.N + ntiles - 1) / ntiles + kIdxSub - 1) / kIdxSub * kIdxSub;
    dim3 grid((a.N + b.key_tile - 1) / b.key_tile, qblocks);
    if (shape_id == 0)
        hipLaunchKernelGGL((indexer_prefill_kernel<32, 128>), grid, dim3(kIdxThreads), 0, s, b);
    else
        hipLaunchKernelGGL((indexer_prefill_kernel<4, 32>), grid, dim3(kIdxThreads), 0, s, b);
    return hipGetLastError();
}

hipError_t launch_indexer_decode(int shape_id, const uint16_t* qI, const uint16_t* kI,
                                 const float* w, float* S, const SeqMeta& m, int blocks,
                                 hipStream_t s) {
    if (blocks <= 0) return hipSuccess;
    if (shape_id == 0)
        hipLaunchKernelGGL((indexer_decode_kernel<32, 128>), dim3(blocks), dim3(kIdxdWaves * 64), 0, s,
                           qI, kI, w, S, m);
    else
        hipLaunchKernelGGL((indexer_decode_kernel<4, 32>), dim3(blocks), dim3(kIdxdWaves * 64), 0, s,
                           qI, kI, w, S, m);
    return hipGetLastError();
}

}  // namespace dsa
