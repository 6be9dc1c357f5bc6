// The main tile GEMM for K-contiguous operands ("NT": A row-major M x K, B
// stored N x K -- the transpose_B form of the local GEMMs in the
// "project_analysis.md" note on TileScale, SUMMA and Cannon examples), the
// layout of the bf16 and fp8 workloads.
//
// Dataflow of the single-GPU GEMM skeleton in "TileScale 与 TileLang比较"
// (section 核心抽象与编程模型对比), mapped onto CDNA4:
//
//  * grid of output tiles: one workgroup of WM x WN waves per BM x BN tile,
//    ordered XCD-aware (tile_coords);
//  * global -> shared copy: buffer loads that write LDS directly (no
//    registers, no ds_write), 16 bytes per lane, 8 rows of 128 bytes per wave
//    instruction, into XOR-swizzled rows; tails need no branches: rows past
//    M or N and 16-byte chunks past K read through an out-of-range offset,
//    which the buffer unit returns as zeros (such rows only feed outputs that
//    are never stored);
//  * pipelined K loop: a ring of NH LDS half-stages (one holds the A rows or
//    the B rows of one K step: RB bytes of K per row); half-stage h is A of
//    step h/2 for even h and B of step h/2 for odd h.  Each K step frees two
//    half-stages and refills them (copies spread between the MFMAs, so the
//    in-order issue never blocks on a full address FIFO).  NH = 4 is two
//    full stages; NH = 5 gives the A rows most of a further step to land;
//  * tile GEMM into register fragments: LDS -> VGPR fragments double-buffered
//    across the K sub-steps (the reads of sub-step s+1 are in flight while
//    the MFMAs of sub-step s run), 32x32 MFMAs accumulating in fp32 AGPRs;
//    the one barrier per K step sits before the last sub-step's MFMAs, which
//    hide its skew and the first reads of the next step;
//  * epilogue: scale (fp8), round to the output type, staged through LDS so
//    that every store instruction writes whole 128-byte lines;
//  * a row-major (N-contiguous) B is taken too (BL = B_NCONTIG): its
//    half-stage holds the step's k rows of the tile's columns, and each B
//    fragment comes from transposing LDS reads (ds_read_b64_tr_b16 for
//    16-bit elements, ds_read_b64_tr_b8 for fp8).
#pragma once

#include <type_traits>

#include "tg_kernels.hpp"

namespace tg {

// offset beyond any valid byte of a buffer resource whose num_records is kNumRecords
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int32_t kNumRecords = 0x7FFFFFF0;
constexpr int32_t kBufferFlags = 0x00020000;  // gfx9 raw buffer, 32-bit data format

typedef __attribute__((address_space(3))) uint8_t* lds_u8_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (wave-uniform): base, stride 0, num_records, flags.
__device__ __forceinline__ i32x4_t make_rsrc(const void* base)
{
    const uint64_t a = (uint64_t)base;
    return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                   __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF), kNumRecords, kBufferFlags};
}

__device__ __forceinline__ uint32_t lds_addr(uint8_t* p)
{
    return (uint32_t)(uintptr_t)(lds_u8_t)p;
}

// One wave instruction: 64 lanes x 16 bytes from global memory straight into
// the 1 KiB of LDS at `dst` (lane i lands at dst + 16*i).  Issued from inline
// assembly so that the compiler does not track it: it would otherwise wait
// for every outstanding copy before each LDS read, and it does not order the
// copies of other waves anyway.  The kernel waits for its copies explicitly
// (wait_copies) before the barrier that publishes them.
__device__ __forceinline__ void load_lds_1k(i32x4_t r, uint8_t* dst, uint32_t voff, uint32_t soff)
{
    // M0 carries the LDS destination; one wait state between writing M0 and the copy
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)),
                   "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr(dst)))
                 : "memory");
}

// As load_lds_1k, with the destination given as an LDS address (wave-uniform):
// no pointer conversion in the hot loop.
__device__ __forceinline__ void load_lds_1k_at(i32x4_t r, uint32_t dst, uint32_t voff, uint32_t soff)
{
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(soff), "{m0}"(dst)
                 : "memory");
}

// As load_lds_1k_at, with the non-temporal hint: for data read once (a
// weight matrix streamed by the skinny GEMM).  Measured on a 128 MiB read
// in the skinny kernel's order: 22.0 us against 24.0 with plain copies.
// Repeated non-temporal reads of one 32 MiB buffer ran at HBM speed where
// plain ones ran twice as fast from the Infinity Cache, so data that other
// workgroups read again soon must not take the hint.  (The assembler takes
// the cache-policy bit only before `lds`.)
__device__ __forceinline__ void load_lds_1k_nt_at(i32x4_t r, uint32_t dst, uint32_t voff, uint32_t soff)
{
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :
                 : "v"(voff), "s"(r), "s"(soff), "{m0}"(dst)
                 : "memory");
}

// wait until at most N of this wave's copies are outstanding (they retire in order)
template <int N>
__device__ __forceinline__ void wait_copies()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// WM x WN waves share the tile (each computes a BM/WM x BN/WN sub-tile).
// With 8 waves (two per SIMD) the LDS sustains about twice the fragment-read
// rate of 4 waves (one per SIMD), which the 256 x 256 tile needs.
template <int E, int O, int BM, int BN, int RB, int NH, int WM = 2, int WN = 2, int BL = B_KCONTIG>
__global__ __launch_bounds__(64 * WM * WN) void gemm_nt(TileArgs p)
{
    constexpr int EB = ElemInfo<E>::bytes;
    constexpr int CE = 16 / EB;       // elements per 16-byte chunk
    constexpr int KE = RB / EB;       // K elements per step
    constexpr int CH = RB / 16;       // 16-byte chunks per staged row
    constexpr int RPI = 1024 / RB;    // rows per copy instruction (64 lanes x 16 bytes)
    constexpr int RSW = 256 / RB;     // rows per 256-byte line of the 64 LDS banks
    constexpr int NW = WM * WN;        // waves
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    constexpr int AI = BM / (NW * RPI), BI = BN / (NW * RPI);  // copy instructions per wave per step
    static_assert(AI >= 1 && BI >= 1 && (BM / NW) % (RSW * CH) == 0 && (BN / NW) % (RSW * CH) == 0 &&
                  (BM / WM) % (RSW * CH) == 0 && (BN / WN) % (RSW * CH) == 0,
                  "wave row blocks must start on a swizzle period");
    // One half-stage slot holds the A rows or the B rows of a K step.  With an
    // even ring depth half-stage h always lands in a slot of h's parity, so
    // the A slots (even) and B slots (odd) take their own sizes (a 256 x 128
    // tile: 32 and 16 KiB, six half-stages in 144 KiB); with an odd depth
    // every slot takes the larger size.
    constexpr int ASZ = BM * RB, BSZ = BN * RB;
    constexpr int HALF = (BM > BN ? BM : BN) * RB;
    constexpr int LDS_BYTES = NH % 2 == 0 ? NH / 2 * (ASZ + BSZ) : NH * HALF;
    static_assert(NH % 2 == 0 || BM == BN, "odd ring depths take square tiles");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    // byte offset of half-stage h's slot
    auto slot_of = [](int64_t h) __attribute__((always_inline)) -> uint32_t {
        const uint32_t i = (uint32_t)h % (uint32_t)NH;  // (h >= 0, below 2^31)
        if constexpr (NH % 2 == 0)
            return (i / 2u) * (uint32_t)(ASZ + BSZ) + (i & 1u) * (uint32_t)ASZ;
        else
            return i * (uint32_t)HALF;
    };
    constexpr int KSTEPS = (E == E_FP8) ? RB / 64 : RB / 32;  // MFMAs along K per step
    static_assert(KSTEPS >= 2 && KSTEPS % 2 == 0, "fragment slots alternate within a step");
    // copy instructions of half-stage h (A rows for even h, B rows for odd h),
    // and of the half-stages h0 .. h1-1 together (the copy waits below)
    auto copies_in = [](int h0, int h1) constexpr {
        int n = 0;
        for (int h = h0; h < h1; ++h)
            n += (h & 1) ? BI : AI;
        return n;
    };
    static_assert(NH >= 4 && copies_in(2, NH - 1) <= 63, "copies in flight");
    typedef typename Mfma32<E>::frag Frag;
    // N-contiguous B (row-major K x N): a B half-stage holds the step's KE
    // rows of k, each BN elements wide (RBN bytes, CHN chunks; the same HALF
    // bytes), copied RPIN rows per instruction and read by the transposing
    // LDS load (16-bit elements only)
    constexpr bool NB = BL == B_NCONTIG;
    constexpr int RBN = BN * EB, CHN = RBN / 16, RPIN = 1024 / RBN;
    static_assert(!NB || (KE * RBN == BN * RB && CHN >= 8 && (KE / RPIN) % NW == 0 && KE / RPIN / NW == BI),
                  "N-contiguous B stage: same size and copy count as the K-contiguous one");
    // physical chunk of logical chunk c of B row k is c ^ swn(k).  16-bit:
    // the four rows k .. k+3 that one transposing read takes (32 bytes each,
    // two 16-lane groups side by side) fall in distinct banks.  8-bit: each
    // half-wave of a transposing read takes 16 bytes of each of 8 rows
    // k .. k+7 in logical chunk c (c even) and 8 more in chunk c ^ 1; with
    // swn even, rows k .. k+7 of chunk c land on the 8 even chunk positions
    // and those of chunk c ^ 1 on the 8 odd ones: 256 bytes, every bank once.
    auto swn = [](uint32_t k) __attribute__((always_inline)) -> uint32_t {
        if constexpr (EB == 1) {
            if constexpr (CHN >= 16)
                return 2u * (k % 8u);
            else
                return 2u * ((k / 2u) % 4u);  // 128-byte rows: two rows per bank line
        } else if constexpr (CHN >= 16) {
            return 4u * (k % 4u);
        } else {
            return 4u * ((((k % 4u) + 1u) / 2u) % 2u);  // 128-byte rows: two rows per bank line
        }
    };

    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps LDS bases scalar
    const int64_t M = p.M, N = p.N, K = p.K;
    const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
    const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
    // K split over S workgroups per tile (S = 1: none); this workgroup runs
    // K steps [kt0, kt0 + NK).  The ring below counts steps from kt0; global
    // offsets use the absolute step kt0 + kt.  With p.dp > 0 the first p.dp
    // workgroups take the first p.dp tiles of the walk whole (one round of
    // the chip) and the workgroups after them split the remaining tiles, so
    // that a last round of few tiles still fills the compute units; split
    // tiles are numbered from p.dp (`stile`) for their counters and shares.
    uint32_t S = p.splits > 1u ? p.splits : 1u;
    uint32_t tmi, tni, ks = 0u, stile = 0u;
    constexpr bool SUB = BM < 256 || BN < 256;  // (a tile smaller than 256 x 256 can cover parts of one)
    if (SUB && p.sub256 != 0u) {
        // the QM x QN parts of the 256 x 256 tiles from walk position
        // sub256 - 1 on: workgroup j takes part j % Q of tile sub256 - 1 + j / Q
        constexpr uint32_t QM = 256 / BM, QN = 256 / BN, Q = QM * QN;
        static_assert(QM * BM == 256 && QN * BN == 256, "parts of a 256 x 256 tile");
        const uint32_t tm2 = (uint32_t)((M + 255) / 256), tn2 = (uint32_t)((N + 255) / 256);
        const uint32_t j = xcd_remap(blockIdx.x, gridDim.x);
        uint32_t t_m, t_n;
        group_walk(p.sub256 - 1u + j / Q, tm2, tn2, p.group_m, t_m, t_n);
        tmi = t_m * QM + (j % Q) / QN;
        tni = t_n * QN + (j % Q) % QN;
        S = 1u;
        if ((int64_t)tmi * BM >= M || (int64_t)tni * BN >= N)
            return;  // (a part past the bottom or right edge of a partial tile)
    } else if (p.dp == 0u) {
        tile_split_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, S, p.group_m, tmi, tni, ks);
        stile = tmi * tiles_n + tni;
    } else if (blockIdx.x < p.dp) {
        tile_coords(blockIdx.x, p.dp, tiles_m, tiles_n, p.group_m, tmi, tni);
        S = 1u;
        stile = 0u;
    } else {
        const uint32_t R = tiles_m * tiles_n - p.dp;  // tiles split, S workgroups each
        const uint32_t idx = xcd_remap(blockIdx.x - p.dp, gridDim.x - p.dp);
        ks = idx / R;
        stile = idx - ks * R;
        group_walk(p.dp + stile, tiles_m, tiles_n, p.group_m, tmi, tni);
    }
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
    const uint32_t ldab = (uint32_t)(p.lda * EB), ldbb = (uint32_t)(p.ldb * EB);
    const int32_t rows_a = (int32_t)(M - m0 < BM ? M - m0 : BM);
    const int32_t rows_b = (int32_t)(N - n0 < BN ? N - n0 : BN);
    const i32x4_t ra = make_rsrc(p.A + m0 * (int64_t)ldab);
    const i32x4_t rb = make_rsrc(NB ? p.B + n0 * EB : p.B + n0 * (int64_t)ldbb);
    const int64_t KT = (K + KE - 1) / KE;  // K is a multiple of CE on this path
    const int64_t kt0 = KT * ks / S, NK = KT * (ks + 1) / S - kt0;

    // ---- staged layout: row r of a stage operand holds RB bytes of K as CH
    // 16-byte chunks; logical chunk c sits at physical chunk c ^ swz(r), with
    // swz(r) = (r / RSW) % CH, so the 16 lanes that read one chunk column
    // from 16 consecutive rows cover all 64 banks.
    //
    // ---- copy instructions: wave w fills rows [w*BM/4, (w+1)*BM/4) of the A
    // stage (likewise B), RPI rows per instruction; lane i lands at physical
    // chunk i%CH of row i/CH, so it loads logical chunk (i%CH) ^ swz(row):
    // the swizzle is applied on the source side.  For instruction j that is
    // (i%CH) ^ ((4j + (i/CH)/RSW) % CH): one value for even j, one for odd j.
    // The per-lane part of the offset is fixed; the step's K offset and the
    // instruction's row block go into the scalar offset.  Rows past M or N:
    // on edge tiles their lanes read through an out-of-range offset (zeros);
    // they only feed outputs that are never stored.
    const uint32_t lrowi = lane / CH;
    const uint32_t lchunk0 = (lane % CH) ^ ((lrowi / RSW) % CH);
    const uint32_t lchunk1 = (lane % CH) ^ ((4u + lrowi / RSW) % CH);
    const uint32_t va0 = (wave * (BM / NW) + lrowi) * ldab + lchunk0 * 16u;
    const uint32_t va1 = (wave * (BM / NW) + lrowi) * ldab + lchunk1 * 16u;
    uint32_t vb0 = (wave * (BN / NW) + lrowi) * ldbb + lchunk0 * 16u;
    uint32_t vb1 = (wave * (BN / NW) + lrowi) * ldbb + lchunk1 * 16u;
    // N-contiguous B: instruction q of wave w copies k rows (w*BI + q)*RPIN
    // + lane/CHN, lane i landing at physical chunk i%CHN of its row, which
    // holds logical chunk (i%CHN) ^ swn(row) (columns 8c .. 8c+7 of the
    // tile); the row's parity class mod 4 alternates with q only, so there
    // is again one offset for even q and one for odd q.  Columns past N read
    // zeros (N is a multiple of 8: no partial chunks).
    const uint32_t lrown = lane / CHN;
    if constexpr (NB) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint32_t kr = (wave * BI + q) * RPIN + lrown;
            const uint32_t lc = (lane % CHN) ^ swn(kr);
            const uint32_t v = lrown * ldbb + lc * 16u;
            const uint32_t oob = n0 + (int64_t)lc * CE < N ? 0u : kOutOfRange;
            (q == 0 ? vb0 : vb1) = v | oob;
        }
    }

    // half-stage of A (or B) of K step kt
    auto a_ptr = [&](int64_t kt) __attribute__((always_inline)) -> uint8_t* {
        return lds + slot_of(2 * kt);
    };
    auto b_ptr = [&](int64_t kt) __attribute__((always_inline)) -> uint8_t* {
        return lds + slot_of(2 * kt + 1);
    };
    auto chunk_oob = [&](int64_t kt, uint32_t lchunk) __attribute__((always_inline)) -> uint32_t {
        // a chunk at or past K (only in the last step) reads through an
        // out-of-range offset (bit 31 set): zeros.  Valid offsets stay below 2^31.
        const int64_t kleft = K - kt * KE;
        const uint32_t kmax = kleft >= KE ? (uint32_t)KE : (uint32_t)kleft;
        return (lchunk * CE < kmax) ? 0u : kOutOfRange;
    };
    // Per-lane offsets of the copies of half-stage h (o0 for even copy
    // instructions, o1 for odd ones), computed once per half-stage.  A step
    // past the last one reads through the out-of-range offset (zeros, into a
    // stage buffer that is not read again).  The K tail is checked only on
    // the edge path: the full-tile path runs with K a multiple of KE.
    auto half_offs = [&](auto edge, int64_t h, uint32_t& o0, uint32_t& o1) __attribute__((always_inline)) {
        const int64_t kt = h >> 1;
        o0 = (h & 1) ? vb0 : va0;
        o1 = (h & 1) ? vb1 : va1;
        if constexpr (decltype(edge)::value) {
            if (!(NB && (h & 1))) {  // (N-contiguous B: the K tail is a row check, in copy_half)
                o0 |= chunk_oob(kt0 + kt, lchunk0);
                o1 |= chunk_oob(kt0 + kt, lchunk1);
            }
        }
        const uint32_t past = kt < NK ? 0u : kOutOfRange;
        o0 |= past;
        o1 |= past;
    };
    // LDS address of this wave's rows in half-stage h
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
    auto half_dst = [&](int64_t h) __attribute__((always_inline)) -> uint32_t {
        return lds0 + slot_of(h) + wave * ((h & 1) ? BN / NW : BM / NW) * RB;
    };
    // copy instruction q of half-stage h (A of step h/2 for even h, B for odd
    // h), with the offsets o0/o1 of that half-stage
    auto copy_half = [&](auto edge, int64_t h, int q, uint32_t o0, uint32_t o1) __attribute__((always_inline)) {
        const int64_t kt = kt0 + (h >> 1);  // absolute K step
        uint32_t v = (q & 1) ? o1 : o0;
        if (NB && (h & 1)) {  // k rows (w*BI + q)*RPIN + lane/CHN of step kt
            const uint32_t kr = (wave * BI + (uint32_t)q) * RPIN;
            if constexpr (decltype(edge)::value)
                v |= kt * KE + kr + lrown < K ? 0u : kOutOfRange;
            load_lds_1k_at(rb, half_dst(h) + q * 1024, v, ((uint32_t)kt * KE + kr) * ldbb);
            return;
        }
        if constexpr (decltype(edge)::value) {
            const int32_t rows = (h & 1) ? rows_b : rows_a;
            v |= (int32_t)(wave * ((h & 1) ? BN / NW : BM / NW) + RPI * q + lrowi) < rows ? 0u : kOutOfRange;
        }
        load_lds_1k_at((h & 1) ? rb : ra, half_dst(h) + q * 1024, v,
                       (uint32_t)kt * RB + (uint32_t)(RPI * q) * ((h & 1) ? ldbb : ldab));
    };

    // ---- fragment reads: every fragment row of this lane has the same swz(row)
    const uint32_t wm = wave / WN, wn = wave % WN;
    const uint32_t lrow = lane & 31u, lgrp = lane >> 5;
    const uint32_t sw = (lrow / RSW) % CH;
    const uint32_t a_row0 = (wm * (BM / WM) + lrow) * RB;
    const uint32_t b_row0 = (wn * (BN / WN) + lrow) * RB;

    Frag fa[2][TM], fb[2][TN];
    // fragment read r (0 .. TM+TN-1) of sub-step s of K step kt into slot
    // `slot`, numbered in the order the MFMAs consume them: A row block 0,
    // every B column block, then A row blocks 1 .. TM-1
    auto read_frag = [&](int64_t kt, int s, int slot, int r) __attribute__((always_inline)) {
        const bool is_a = (r == 0) || (r > TN);
        const int idx = (r == 0) ? 0 : (r <= TN ? r - 1 : r - TN);
        const uint8_t* st = is_a ? a_ptr(kt) : b_ptr(kt);
        const uint32_t row0 = (is_a ? a_row0 : b_row0) + (uint32_t)idx * 32 * RB;
        Frag f;
        if constexpr (NB && EB == 1) {
            if (!is_a) {
                // 32 k of column n of the block from four transposing reads (8
                // k each): in each 16-lane group, source lane 2e + a addresses
                // k row (base + e), columns 8a .. 8a+7 of the group's 16, and
                // lane 8a + j receives column 8a + j at rows base .. base+7
                const uint32_t l16 = lane % 16u;
                const uint32_t col = wn * (BN / WN) + (uint32_t)idx * 32u + 16u * ((lane / 16u) % 2u) + 8u * (l16 % 2u);
                // rows k0 + 8*r2 share swn(k0) (same k % 8): one address, the
                // four reads 8 rows apart
                const uint32_t k0 = (uint32_t)(64 * s) + 32u * lgrp + l16 / 2u;
                const uint32_t off = k0 * RBN + (((col / CE) ^ swn(k0)) << 4) + (col % CE);
                uint32_t w[8];
#pragma unroll
                for (int r2 = 0; r2 < 4; ++r2) {
                    const v2i32_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) v2i32_t*)(lds_u8_t)(st + off + (uint32_t)r2 * 8u * RBN));
                    w[2 * r2] = (uint32_t)v[0];
                    w[2 * r2 + 1] = (uint32_t)v[1];
                }
                f = i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
            } else {
                const uint32_t c0 = (uint32_t)(4 * s) + 2u * lgrp;
                const u32x4 lo = lds128(st, row0 + ((c0 ^ sw) << 4));
                const u32x4 hi = lds128(st, row0 + (((c0 + 1u) ^ sw) << 4));
                f = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
        } else if constexpr (NB) {
            if (!is_a) {
                // 8 k of column n of the block from two transposing reads (4 k
                // each): in each 16-lane group, source lane 4e + a addresses k
                // row (base + e), columns 4a .. 4a+3 of the group's 16, and lane
                // 4a + j receives column 4a + j at rows base .. base+3
                const uint32_t l16 = lane % 16u;
                const uint32_t col = wn * (BN / WN) + (uint32_t)idx * 32u + 16u * ((lane / 16u) % 2u) + 4u * (l16 % 4u);
                uint32_t w[4];
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2) {
                    const uint32_t k = (uint32_t)(16 * s) + 8u * lgrp + 4u * (uint32_t)r2 + l16 / 4u;
                    const uint32_t off = k * RBN + (((col / CE) ^ swn(k)) << 4) + (col % CE) * EB;
                    const auto v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(lds_u8_t)(st + off));
                    w[2 * r2] = (uint32_t)(uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
                    w[2 * r2 + 1] = (uint32_t)(uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
                }
                f = u32x4{w[0], w[1], w[2], w[3]};
            } else {
                f = lds128(st, row0 + ((((uint32_t)(2 * s) + lgrp) ^ sw) << 4));
            }
        } else if constexpr (E == E_FP8) {
            const uint32_t c0 = (uint32_t)(4 * s) + 2u * lgrp;
            const u32x4 lo = lds128(st, row0 + ((c0 ^ sw) << 4));
            const u32x4 hi = lds128(st, row0 + (((c0 + 1u) ^ sw) << 4));
            f = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        } else {
            f = lds128(st, row0 + ((((uint32_t)(2 * s) + lgrp) ^ sw) << 4));
        }
        if (is_a)
            fa[slot][idx] = f;
        else
            fb[slot][idx] = f;
    };
    auto read_frags = [&](int64_t kt, int s, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < TM + TN; ++r)
            read_frag(kt, s, slot, r);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{};

    // acc[i][j] holds the transposed 32x32 block (B rows x A rows): value v of
    // lane l is C[m = i*32 + l%32][n = j*32 + 8*(v/4) + 4*(l/32) + v%4], so every
    // lane owns runs of 4 consecutive output columns.
    //
    // One sub-step: the TM*TN MFMAs of fragment slot `slot`.  The fragment
    // reads of the next sub-step and the NQ copy instructions (from the first
    // MFMA on, so they get the most time to land) sit between the MFMAs, each
    // pinned in place: the wave's in-order issue never waits on a burst of
    // LDS reads or on a full address queue.  The reads are spread over all
    // the MFMAs, except on the 16-bit 256 x 256 tile with its four-slot ring
    // (two waves per SIMD), where over the first half ran ~2% faster at
    // 4096^3 .. 8192^3 (and 1-3% slower on the other tiles and rings).
    constexpr int NT = TM * TN, NR = TM + TN;
    constexpr bool FRONT = E != E_FP8 && BM == 256 && BN == 256 && NH == 4;
    auto substep = [&](int slot, auto rd, auto cp, auto nq) __attribute__((always_inline)) {
        constexpr int NQ = decltype(nq)::value;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int i = t / TN, j = t % TN;
            acc[i][j] = Mfma32<E>::run(fb[slot][j], fa[slot][i], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (FRONT ? r * (NT / 2) / NR == t : r * NT / NR == t)
                    rd(r);
            if constexpr (NQ > 0) {
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    if (q * NT / NQ == t)
                        cp(q);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto nothing = [](int) {};

    // One K step.  Entering, the fragments of its sub-step 0 are in slot 0.
    // Half-stage 2kt+NH-1 (whose slot was freed by the previous barrier) is
    // copied during sub-step 0.  The barrier before the last sub-step
    // publishes step kt+1 (half-stages past 2kt+3 may still be in flight) and
    // frees the two half-stages of step kt: half-stage 2kt+NH is copied during
    // the last sub-step, while the first fragments of step kt+1 are read.
    auto step = [&](auto edge, int64_t kt) __attribute__((always_inline)) {
        uint32_t p0, p1, r0, r1;
        half_offs(edge, 2 * kt + NH - 1, p0, p1);
        half_offs(edge, 2 * kt + NH, r0, r1);
#pragma unroll
        for (int s = 0; s < KSTEPS - 1; ++s) {
            auto rd = [&](int r) __attribute__((always_inline)) { read_frag(kt, s + 1, (s + 1) & 1, r); };
            // (the half-stage freed by the last barrier is copied during the
            // first sub-step; with an odd ring depth, where that is an A
            // half-stage, during the second: 1-4% faster at 3072^3 .. 3584^3)
            if (s == ((NH & 1) && KSTEPS > 2 ? 1 : 0))
                substep(s & 1, rd,
                        [&](int q) __attribute__((always_inline)) { copy_half(edge, 2 * kt + NH - 1, q, p0, p1); },
                        std::integral_constant<int, ((NH - 1) & 1) ? BI : AI>{});
            else
                substep(s & 1, rd, nothing, std::integral_constant<int, 0>{});
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_copies<copies_in(4, NH)>();  // own copies of step kt+1 landed ...
        __syncthreads();               // ... and every wave's; the half-stages of step kt are free
        __builtin_amdgcn_sched_barrier(0);
        // (the reads of step kt+1 after the last step are stale and unused)
        substep((KSTEPS - 1) & 1, [&](int r) __attribute__((always_inline)) { read_frag(kt + 1, 0, 0, r); },
                [&](int q) __attribute__((always_inline)) { copy_half(edge, 2 * kt + NH, q, r0, r1); },
                std::integral_constant<int, (NH & 1) ? BI : AI>{});
    };

    auto run = [&](auto edge) __attribute__((always_inline)) {
        // half-stages 0 .. NH-2
#pragma unroll
        for (int h = 0; h < NH - 1; ++h) {
            uint32_t o0, o1;
            half_offs(edge, h, o0, o1);
#pragma unroll
            for (int j = 0; j < ((h & 1) ? BI : AI); ++j)
                copy_half(edge, h, j, o0, o1);
        }
        wait_copies<copies_in(2, NH - 1)>();  // step 0 landed
        __syncthreads();
        read_frags(0, 0, 0);
        for (int64_t kt = 0; kt < NK; ++kt)
            step(edge, kt);
        wait_copies<0>();  // copies past the last step (zeros) must land before LDS is reused
    };
    if (NK > 0) {
        if (rows_a == BM && rows_b == BN && K % KE == 0)  // full tiles, no K tail
            run(std::false_type{});
        else
            run(std::true_type{});
    }
    mfma_drain();
    __syncthreads();  // every wave is done reading the stage buffers (the epilogue reuses them)

    // ---- K split: store this wave's partial share, count in; the last of the
    // S arrivals adds the S partials in split order and goes on to store the
    // share, the others are done.  (No barrier follows: each wave stages its
    // share in its own LDS region.)
    if (S > 1u) {
        constexpr int SHARE = TM * TN * 1024;  // floats of a wave's share
        const uint32_t tile = stile;
        float* const share0 = p.partials + ((size_t)tile * S * NW + wave) * SHARE;  // split 0's slot
        auto slot = [&](uint32_t q) __attribute__((always_inline)) { return share0 + (size_t)q * NW * SHARE; };
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    splitk_store(slot(ks), i * TN + j, g, lane,
                                 f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]});
        if (!splitk_last(p.counters + (size_t)tile * NW + wave, S, lane))
            return;
        // the S partial shares in split order: acc = p_0, then acc += p_q
        // for q = 1 .. S-1.  Up to 4 accumulator blocks per wave (the 64 and
        // 128 tiles), this wave's own share p_ks is taken from the
        // accumulator itself (the bits it stored) and the other shares are
        // loaded whole, several at a time up to 64 floats per lane, all of a
        // batch's loads ahead of its adds.  With more blocks (the 256 tile,
        // which the planner never splits) the own share is read back like
        // the others, two blocks at a time, to keep the registers in bounds.
        constexpr int NBLK = TM * TN;
        if constexpr (NBLK <= 4) {
            constexpr int QB = 4 / NBLK;  // shares per batch
            f32x4 own[NBLK][4];
#pragma unroll
            for (int b = 0; b < NBLK; ++b)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    own[b][g] = f32x4{acc[b / TN][b % TN][4 * g], acc[b / TN][b % TN][4 * g + 1],
                                      acc[b / TN][b % TN][4 * g + 2], acc[b / TN][b % TN][4 * g + 3]};
            for (uint32_t q0 = 0; q0 < S; q0 += QB) {
                f32x4 v[QB][NBLK][4];
#pragma unroll
                for (int qq = 0; qq < QB; ++qq) {
                    const uint32_t q = q0 + (uint32_t)qq;
                    if (q < S && q != ks)
#pragma unroll
                        for (int b = 0; b < NBLK; ++b)
#pragma unroll
                            for (int g = 0; g < 4; ++g)
                                v[qq][b][g] = splitk_load(slot(q), b, g, lane);
                }
#pragma unroll
                for (int qq = 0; qq < QB; ++qq) {
                    const uint32_t q = q0 + (uint32_t)qq;
                    if (q < S) {
#pragma unroll
                        for (int b = 0; b < NBLK; ++b)
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                const f32x4 x = q == ks ? own[b][g] : v[qq][b][g];
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    acc[b / TN][b % TN][4 * g + e] =
                                        q == 0u ? x[e] : acc[b / TN][b % TN][4 * g + e] + x[e];
                            }
                    }
                }
            }
        } else {
            constexpr int BB = 2;
            for (uint32_t q = ks == 0u ? 1u : 0u; q < S; ++q) {
                const float* src = slot(q);
#pragma unroll
                for (int b0 = 0; b0 < NBLK; b0 += BB) {
                    f32x4 v[BB][4];
#pragma unroll
                    for (int bb = 0; bb < BB; ++bb)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            v[bb][g] = splitk_load(src, b0 + bb, g, lane);
#pragma unroll
                    for (int bb = 0; bb < BB; ++bb) {
                        const int i = (b0 + bb) / TN, j = (b0 + bb) % TN;
#pragma unroll
                        for (int g = 0; g < 4; ++g)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                acc[i][j][4 * g + e] = q == 0u ? v[bb][g][e] : acc[i][j][4 * g + e] + v[bb][g][e];
                    }
                }
            }
        }
    }

    // ---- epilogue
    constexpr int WR = BM / WM, WC = BN / WN;  // this wave's sub-tile
    const int64_t wrow0 = m0 + wm * WR, wcol0 = n0 + wn * WC;
    auto out_val = [&](int i, int j, int v) __attribute__((always_inline)) -> float {
        float x = acc[i][j][v];
        if constexpr (E == E_FP8)
            x *= p.alpha;
        return x;
    };
    if constexpr (O == O_F32) {
        // fp32 output: staged through LDS like the 16-bit one, so that the
        // stores are whole rows (a lane's 4 columns stored directly give 32
        // rows x 32 bytes per instruction, which measured ~50% slower for the
        // whole 4096^3 GEMM).  The wave's sub-tile takes 4*WC bytes per row,
        // so it goes in passes of PR rows.
        constexpr int OB = WC * 4;            // bytes per staged output row
        constexpr int NCH = OB / 16;          // 16-byte chunks per row
        constexpr int PBY = LDS_BYTES / NW;   // staging bytes per wave
        // rows per pass: the largest of WR, WR/2, WR/4 that fits
        constexpr int PR = PBY / OB >= WR ? WR : (PBY / OB >= WR / 2 ? WR / 2 : WR / 4);
        static_assert(PR % 32 == 0 && WR % PR == 0 && (PR * NCH) % 64 == 0, "fp32 staging passes");
        uint8_t* ep = lds + wave * PBY;
        float* C = (float*)p.C;
#pragma unroll
        for (int pass = 0; pass < WR / PR; ++pass) {
#pragma unroll
            for (int ii = 0; ii < PR / 32; ++ii) {
                const int i = pass * (PR / 32) + ii;
                const uint32_t r = ii * 32 + lrow;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const uint32_t c = (uint32_t)(8 * j + 2 * g) + lgrp;  // chunk of columns j*32 + 8g + 4*lgrp .. +3
                        const f32x4 q = {out_val(i, j, 4 * g), out_val(i, j, 4 * g + 1), out_val(i, j, 4 * g + 2),
                                         out_val(i, j, 4 * g + 3)};
                        *(f32x4*)(ep + r * OB + ((c ^ (r % NCH)) << 4)) = q;
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes done
#pragma unroll
            for (int t = 0; t < PR * NCH / 64; ++t) {
                const uint32_t idx = t * 64 + lane;
                const uint32_t r = idx / NCH, c = idx % NCH;
                const f32x4 q = bit_cast<f32x4>(lds128(ep, r * OB + ((c ^ (r % NCH)) << 4)));
                const int64_t row = wrow0 + pass * PR + r, col = wcol0 + c * 4;
                if (row < M) {
                    if (col + 4 <= N) {
                        store_nt((f32x4*)(C + row * p.ldc + col), q);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (col + e < N)
                                C[row * p.ldc + col + e] = q[e];
                    }
                }
            }
        }
    } else {
        // 16-bit output: each wave stages its sub-tile in its own LDS region
        // (row-major, 16-byte chunks XOR-swizzled by row), then writes whole
        // rows with 16-byte stores.
        constexpr int OB = WC * 2;          // bytes per staged output row
        constexpr int NCH = OB / 16;        // 16-byte chunks per row
        constexpr int WBYTES = WR * OB;     // bytes per wave
        static_assert(NW * WBYTES <= LDS_BYTES, "epilogue staging must fit the stage buffers");
        uint8_t* ep = lds + wave * WBYTES;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint32_t r = i * 32 + lrow;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t c = (uint32_t)(4 * j + g);  // 16-byte chunk of columns j*32 + 8g .. +7
                    const uint32_t lo = (uint32_t)convert_out<O>(out_val(i, j, 4 * g)) |
                                        ((uint32_t)convert_out<O>(out_val(i, j, 4 * g + 1)) << 16);
                    const uint32_t hi = (uint32_t)convert_out<O>(out_val(i, j, 4 * g + 2)) |
                                        ((uint32_t)convert_out<O>(out_val(i, j, 4 * g + 3)) << 16);
                    *(u32x2*)(ep + r * OB + ((c ^ (r % NCH)) << 4) + lgrp * 8) = u32x2{lo, hi};
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes done
        uint16_t* C = (uint16_t*)p.C;
#pragma unroll
        for (int t = 0; t < WR * NCH / 64; ++t) {
            const uint32_t idx = t * 64 + lane;
            const uint32_t r = idx / NCH, c = idx % NCH;
            const u32x4 q = lds128(ep, r * OB + ((c ^ (r % NCH)) << 4));
            const int64_t row = wrow0 + r, col = wcol0 + c * 8;
            if (row < M) {
                if (col + 8 <= N) {
                    store_nt((u32x4*)(C + row * p.ldc + col), q);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (col + e < N)
                            C[row * p.ldc + col + e] = (uint16_t)(q[e >> 1] >> ((e & 1) * 16));
                }
            }
        }
    }
}

}  // namespace tg
