// The GEMM for M <= 16 rows against a K-contiguous B (decode-shaped products:
// a few activation rows against a weight stored N x K); batches of a few
// times 16 rows run one workgroup per 16-row slice.  Streaming B from
// HBM is the whole cost.  The waves of a workgroup split K and reduce their
// partial tiles through LDS -- the intra-block split-K of the TileScale
// README's GEMM example (section "Example of GEMM"), where warpgroups split
// K and all-reduce on chip.
//
// Each workgroup owns 16 or 32 columns (B rows).  Each wave streams its K
// range through a private LDS ring of RING slots with direct-to-LDS copies; a
// slot holds one stage of 64 k: 128 bytes of each of the B rows and of the A
// rows.  One copy instruction fetches 8 rows x 128 bytes -- whole cache lines
// -- which the memory system streams faster than the 16 rows x 64 bytes a
// lane-per-operand register load would fetch.  Chunks are XOR-swizzled by
// row so the fragment reads are free of bank conflicts.  A wave waits only
// for its own copies (no barrier in the loop); with RING = 2 the copies of
// stage s+1 are in flight while stage s is multiplied, which measured faster
// than deeper rings (more requests in flight stream no faster).
//
// MFMA: 16x16x32 with the operands swapped (B rows in the first operand):
// lane l supplies 8 k of B column l%16 and of A row l%16 (rows past M read
// as zeros), lane quarter h = l/16 takes k = 8h .. 8h+7 of each 32.  The
// result lane l, value v is row l%16, column 4*(l/16) + v.
//
// A K tail (K % 64) is multiplied after the ring by one wave, from global
// memory with element masks.
#pragma once

#include "tg_gemm_nt.hpp"

namespace tg {

constexpr int kSkKE = 64;     // k per stage
constexpr int kSkRow = 128;   // bytes per staged row (16-bit elements)

// Slot bytes: the 16*CG B rows, then 8*AI A rows (AI copy instructions).
template <int AI, int CG> struct SkinnySlot {
    static constexpr int BYTES = (16 * CG + 8 * AI) * kSkRow;
};

// physical 16-byte chunk of logical chunk c of staged row r: two rows share
// a 256-byte line of the 64 banks, so 16 rows at one logical chunk land in 16
// distinct bank groups
__device__ __forceinline__ uint32_t sk_swz(uint32_t r, uint32_t c)
{
    return c ^ ((r >> 1) & 7u);
}

// SPLIT: the K stages are also split over gridDim.y workgroups per column
// block (for narrow N, where N / 16 workgroups leave CUs idle).
//   SPLIT = 1: each adds its partial tile into the fp32 output, which the
//              host has zeroed (fp32 atomic adds: the summation order over
//              the split is not fixed);
//   SPLIT = 2: each stores its partial tile in a workspace slot and counts
//              in; the last to arrive adds the partials in split order (a
//              fixed order) and stores C, of any output type (splitk_last).
//
// CG: 16-column groups per workgroup (16*CG columns).  Every workgroup
// copies its slice's A rows over all of K, so with CG = 2 the A bytes the
// compute units copy halve, for half the workgroups.
template <int E, int O, int WAVES, int AI, int RING, int SPLIT = 0, int CG = 1>
__global__ __launch_bounds__(WAVES * 64) void skinny_gemm(SkinnyArgs p)
{
    typedef typename OutInfo<O>::T OutT;
    static_assert(E == E_F16 || E == E_BF16, "16-bit inputs");
    static_assert(SPLIT != 1 || O == O_F32, "partial tiles are added in fp32");
    constexpr int SLOT = SkinnySlot<AI, CG>::BYTES;
    constexpr int COLS = 16 * CG;          // columns (B rows) per workgroup
    constexpr int BI = COLS / 8;           // B copy instructions per stage
    constexpr int PER = BI + AI;           // copy instructions per stage
    constexpr int ZERO = WAVES * RING * SLOT;  // 16 zero bytes: A rows past 8*AI
    static_assert(AI >= 1 && AI <= 2 && RING >= 2 && (RING - 1) * PER <= 63, "copy ring");
    static_assert(ZERO + 16 <= 160 * 1024 && WAVES * CG * 4 * 64 * 4 <= ZERO, "LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[ZERO + 16];

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t N = p.N, K = p.K;
    // Rows come in slices of 16 (one per workgroup): workgroup id -> (column
    // block, slice) so that the S slices of a column block have ids 8 apart,
    // i.e. run on one XCD at about the same time and share its L2's copy of
    // the block's B rows.  With S = 1 this is the identity.
    const int64_t S = (p.M + 15) / 16;
    const int64_t grp8 = (int64_t)blockIdx.x / (8 * S), rem = (int64_t)blockIdx.x % (8 * S);
    const int64_t slice = rem / 8;
    const int64_t n0 = (grp8 * 8 + rem % 8) * COLS;
    if (n0 >= N)
        return;  // padding of the last group of eight column blocks (whole workgroup)
    const int64_t M = p.M - 16 * slice < 16 ? p.M - 16 * slice : 16;  // rows of this slice
    const uint8_t* const Ab = p.A + 16 * slice * p.lda * 2;
    const int64_t KS = K / kSkKE;  // whole stages
    // this workgroup's stages [z0, z1), split over its waves in contiguous ranges
    const int64_t z0 = SPLIT != 0 ? KS * blockIdx.y / gridDim.y : 0;
    const int64_t z1 = SPLIT != 0 ? KS * (blockIdx.y + 1) / gridDim.y : KS;
    const int64_t s0 = z0 + (z1 - z0) * wave / WAVES;
    const int64_t nst = z0 + (z1 - z0) * (wave + 1) / WAVES - s0;
    if (tid == 0)
        *(u32x4*)(lds + ZERO) = u32x4{0u, 0u, 0u, 0u};

    // Copy lanes: instruction i fetches rows 8i + lane/8; the lane's physical
    // chunk lane%8 holds the row's logical chunk sk_swz(row, lane%8).  Rows
    // past M or N and stages past the wave's range read through an
    // out-of-range offset (zeros).  The host guarantees every valid offset,
    // plus the stage offsets the ring forms, stays below 2^31.
    const i32x4_t ra = make_rsrc(Ab);
    const i32x4_t rb = make_rsrc(p.B + n0 * p.ldb * 2);
    uint32_t vb[BI], va[AI];
#pragma unroll
    for (int i = 0; i < BI; ++i) {
        const uint32_t r = 8u * i + lane / 8u;
        vb[i] = n0 + r < N ? r * (uint32_t)p.ldb * 2u + sk_swz(r, lane % 8u) * 16u : kOutOfRange;
    }
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const uint32_t r = 8u * i + lane / 8u;
        va[i] = (int64_t)r < M ? r * (uint32_t)p.lda * 2u + sk_swz(r, lane % 8u) * 16u : kOutOfRange;
    }
    const uint32_t ring = __builtin_amdgcn_readfirstlane(lds_addr(lds)) + wave * (RING * SLOT);
    // B rows read by this workgroup alone (one slice) stream with the
    // non-temporal hint; with several slices the later ones read them from L2
    // (measured: M = 16 29.2 -> 28.0 us per flushed launch at N = K = 8192;
    // M = 24 and 32 lose 3.5-6 us with it)
    const bool b_once = S == 1;
    auto issue = [&](int64_t st, uint32_t slot) __attribute__((always_inline)) {
        const uint32_t past = st < nst ? 0u : kOutOfRange;
        const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)((s0 + st) * kSkRow));
        if (b_once) {
#pragma unroll
            for (int i = 0; i < BI; ++i)
                load_lds_1k_nt_at(rb, slot + i * 1024, vb[i] | past, soff);
        } else {
#pragma unroll
            for (int i = 0; i < BI; ++i)
                load_lds_1k_at(rb, slot + i * 1024, vb[i] | past, soff);
        }
#pragma unroll
        for (int i = 0; i < AI; ++i)
            load_lds_1k_at(ra, slot + COLS * kSkRow + i * 1024, va[i] | past, soff);
    };

    // two accumulators per column group (the two 32-k halves of a stage)
    f32x4 acc[CG][2];
#pragma unroll
    for (int g = 0; g < CG; ++g)
        acc[g][0] = acc[g][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t c16 = lane & 15u, h = lane >> 4;
    const bool arow = c16 < 8u * AI;  // this lane's A row is held in the slot
    const uint32_t lbase = wave * (RING * SLOT);
    auto compute = [&](uint32_t cur) __attribute__((always_inline)) {
        const uint32_t slot = lbase + cur * SLOT;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint32_t c = 4u * s + h;
            const u32x4 a = lds128(lds, arow ? slot + (COLS + c16) * kSkRow + (sk_swz(c16, c) << 4) : (uint32_t)ZERO);
#pragma unroll
            for (int g = 0; g < CG; ++g) {
                // (rows 16g + c16 share sk_swz with row c16)
                const u32x4 b = lds128(lds, slot + (16u * g + c16) * kSkRow + (sk_swz(c16, c) << 4));
                acc[g][s] = Mfma16<E>::run(b, a, acc[g][s]);
            }
        }
    };

    __syncthreads();  // the zero block is written
    if (nst > 0) {
#pragma unroll
        for (int r = 0; r < RING - 1; ++r)
            issue(r, ring + r * SLOT);
        uint32_t cur = 0;  // slot of stage st
        for (int64_t st = 0; st < nst; ++st) {
            const uint32_t nxt = cur >= 1 ? cur - 1 : RING - 1;  // slot of stage st+RING-1 == slot of st-1
            issue(st + RING - 1, ring + nxt * SLOT);
            wait_copies<(RING - 1) * PER>();  // this wave's copies of stage st have landed
            __builtin_amdgcn_sched_barrier(0);
            compute(cur);
            __builtin_amdgcn_sched_barrier(0);
            cur = cur + 1 == RING ? 0 : cur + 1;
        }
    }
    wait_copies<0>();  // the trailing zero stages land before LDS is reused

    // the K tail (K % 64: at most two 32-wide blocks, the last one partial),
    // taken by one wave of the workgroup that holds the end of K
    if (K % kSkKE != 0 && wave == WAVES - 1 && (SPLIT == 0 || blockIdx.y == gridDim.y - 1)) {
        for (int64_t kb = KS * 2; kb * 32 < K; ++kb) {
            const int64_t k = kb * 32 + h * 8;
            u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if ((int64_t)c16 < M && k < K) {
                const uint8_t* src = Ab + ((int64_t)c16 * p.lda + k) * 2;
                a = (k + 8 <= K) ? ldg128(src) : load_chunk_partial<2>(src, K - k);
            }
#pragma unroll
            for (int g = 0; g < CG; ++g) {
                const int64_t n = n0 + 16 * g + c16;
                b = u32x4{0u, 0u, 0u, 0u};
                if (n < N && k < K) {
                    const uint8_t* src = p.B + (n * p.ldb + k) * 2;
                    b = (k + 8 <= K) ? ldg128(src) : load_chunk_partial<2>(src, K - k);
                }
                acc[g][0] = Mfma16<E>::run(b, a, acc[g][0]);
            }
        }
    }
    mfma_drain();

    // partial tiles: value v of lane l is row l%16, column 16g + 4*(l/16) + v
    __syncthreads();
    float* red = (float*)lds;  // [wave][group][v][lane]
#pragma unroll
    for (int g = 0; g < CG; ++g)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[((wave * CG + g) * 4 + v) * 64 + lane] = acc[g][0][v] + acc[g][1][v];
    __syncthreads();
    if (wave < (uint32_t)CG) {  // wave g sums column group g over the K split, in wave order
        const uint32_t g = wave;
        OutT* C = (OutT*)p.C + 16 * slice * p.ldc;
        const int64_t r = c16;
        f32x4 sum;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            sum[v] = red[(g * 4 + v) * 64 + lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w)
                sum[v] += red[((w * CG + g) * 4 + v) * 64 + lane];
        }
        if constexpr (SPLIT == 2) {
            // this workgroup's partial tile into its slot (1 KiB: one value
            // quadruple per lane), count in; the last of the gridDim.y
            // arrivals adds them in split order, its own from registers (the
            // bits it stored) and the others loaded 8 at a time, all of a
            // batch's loads ahead of its adds
            // (per column group: slots [block][group][split], counter [block][group])
            float* const slot0 = p.partials + ((size_t)blockIdx.x * CG + g) * gridDim.y * 256;
            splitk_store(slot0 + blockIdx.y * 256, 0, 0, lane, sum);
            if (!splitk_last(p.counters + (size_t)blockIdx.x * CG + g, gridDim.y, lane))
                return;
            const f32x4 own = sum;
            const uint32_t S = gridDim.y, me = blockIdx.y;
            for (uint32_t q0 = 0; q0 < S; q0 += 8) {
                f32x4 v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t q = q0 + (uint32_t)j;
                    if (q < S && q != me)
                        v[j] = splitk_load(slot0 + q * 256, 0, 0, lane);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t q = q0 + (uint32_t)j;
                    if (q < S) {
                        const f32x4 x = q == me ? own : v[j];
                        sum = q == 0u ? x : sum + x;
                    }
                }
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t col = n0 + 16 * g + 4 * h + v;
            if (r < M && col < N) {
                if constexpr (SPLIT == 1)
                    atomicAdd((float*)C + r * p.ldc + col, sum[v]);
                else
                    C[r * p.ldc + col] = convert_out<O>(sum[v]);
            }
        }
    }
}

// Whether every buffer offset of skinny_gemm stays below the descriptor's
// range: the largest row offset of A (16 rows) and of a column block of B
// (16 * cg rows), plus the stage offsets the ring forms (up to RING stages
// past the end of K).
inline bool skinny_offsets_fit(int64_t K, int64_t lda, int64_t ldb, int ring, int cg)
{
    const int64_t span = K * 2 + (int64_t)ring * kSkRow + kSkRow;
    const int64_t lim = (int64_t)kNumRecords;
    return 16 * lda * 2 + span < lim && 16 * cg * ldb * 2 + span < lim;
}

}  // namespace tg
