// The w4a16 Dequant-GEMM: fp16 activations x int4 weights (packed 8 per
// int32 along K, one fp16 scale per 128 K per column, a scalar zero point),
// fp32 accumulation, fp16 output.  Dequant-GEMM is one of the target kernels
// of "TileScale 与 TileLang比较" (sections 设计目标、定位与适用场景 and
// 生态互操作、性能、局限与路线图); the tile dataflow is the single-GPU GEMM
// skeleton of the same page (section 核心抽象与编程模型对比).
//
// Built on the NT kernel's machinery (tg_gemm_nt.hpp): A is copied straight
// into an LDS ring with an XOR swizzle and read into MFMA fragments, with
// the same operand swap and staged fp16 epilogue.  B never passes through a
// shared stage: each wave copies its own columns' int4 words into LDS,
// reads them back and dequantises each word with tg::dequant_w4_word -- the
// routine tg_dequant_w4 also runs -- directly into the MFMA operand
// registers, interleaved with the MFMAs.
#pragma once

#include "tg_gemm_nt.hpp"

namespace tg {

// One wave instruction: 64 lanes x 4 bytes from global memory straight into
// the 256 bytes of LDS at `dst` (lane i lands at dst + 4*i).
__device__ __forceinline__ void load_lds_256(i32x4_t r, uint8_t* dst, uint32_t voff, uint32_t soff)
{
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff)),
                   "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr(dst)))
                 : "memory");
}

// Empty instruction that claims to rewrite v: the value becomes available
// (the compiler waits for its load) here, and a loop-carried value set by it
// is not a load that could be re-issued at its use in the next iteration.
template <typename T>
__device__ __forceinline__ void pin(T& v)
{
    asm volatile("" : "+v"(v));
}

// Largest K the kernel takes: the scales of its 128 columns for the whole K
// range are held in LDS (2 bytes per column per 128 K).
constexpr int kW4MaxGroups = 128;  // K <= 16384

// Requirements (checked by the host): K a multiple of 256 and at most
// 128 * kW4MaxGroups, scales 4-byte aligned with an even row stride.
//
// Work split: the workgroup computes a BM x 128 tile with 8 waves, two per
// SIMD.  Waves w and w+4 own columns 32(w%4) .. +31 and all BM rows; wave w
// takes the even K steps and wave w+4 the odd ones, each into its own
// accumulators (BM/32 blocks of 32 x 32), which are summed at the end.  The
// two waves of a SIMD thus share its matrix unit and its VALU: one
// dequantises while the other's MFMAs run.  Each weight is dequantised once,
// by the one wave that multiplies it, straight into the MFMA operand.
//
// A K step is 128 wide (one scale group).  A 32x32x16 MFMA takes, in lane l,
// eight k values of row/column l % 32; lanes 0..31 hold its k slots 0..7,
// lanes 32..63 slots 8..15.  Which k of the step a slot carries is free as
// long as A and B agree, so sub-step s (0..7) gives lane half h the slots
// k = 64h + 8s .. +7: int4 word 8h + s of the column's 16 words of the step,
// and 16-byte chunk 8h + s of the A row's 256 bytes.
//
// Memory requests.  A vector L1 keeps a bounded number of requests to L2 in
// flight, so the kernel moves whole lines where it can: A rows are 256 bytes
// per step; a column's 64 bytes of words per step are fetched by four
// neighbouring lanes of one copy instruction (one request); the scales are
// fetched once, before the K loop.
//
// Ring: NA steps of A and words in LDS, NA/2 per wave group.  The group
// that runs a step also copies it (each of its 4 waves a quarter of A and
// its own columns' words), NA-2 steps ahead: at the barrier that opens
// group step k, the slot of the group's step k-2 is free and is refilled
// with step k+NA-2.
constexpr int kW4Threads = 512;

template <int BM, int NA>
__global__ __launch_bounds__(kW4Threads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_w4(TileArgs p)
{
    constexpr int BN = 128;
    constexpr int RB = 256;          // bytes of K per staged A row: 128 fp16
    constexpr int KE = 128;          // K elements per step
    constexpr int CH = 16;           // 16-byte chunks per staged A row
    constexpr int RPI = 1024 / RB;   // A rows per copy instruction
    constexpr int SUB = 8;           // MFMA sub-steps per step
    constexpr int TM = BM / 32;      // 32-row accumulators per wave
    constexpr int AI = BM / 4 / RPI; // A copy instructions per wave per step
    constexpr int ASTAGE = BM * RB;
    constexpr int WSTAGE = 4 * 2048; // per step: 4 waves x 32 columns x 64 bytes of words
    constexpr int CPS = AI + 2;      // copy instructions per wave per group step
    static_assert(BM % 64 == 0 && NA == 4 && CPS <= 63, "tile / ring of two slots per group");
    typedef u32x4 Frag;

    __shared__ __attribute__((aligned(1024))) uint8_t lds_a[NA * ASTAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_w[NA * WSTAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_s[BN * kW4MaxGroups * 2];

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t grp = wave >> 2, wq = wave & 3u;  // K-step parity; column quarter
    const int64_t M = p.M, N = p.N, K = p.K;
    const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
    const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
    uint32_t tmi, tni;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, p.group_m, tmi, tni);
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
    const uint32_t ldab = (uint32_t)(p.lda * 2);
    const int32_t rows_a = (int32_t)(M - m0 < BM ? M - m0 : BM);
    const int32_t cols_b = (int32_t)(N - n0 < BN ? N - n0 : BN);
    const uint32_t KT = (uint32_t)(K / KE);  // even
    const uint32_t G = (uint32_t)(K / 128);  // scale groups per column
    const i32x4_t ra = make_rsrc(p.A + m0 * (int64_t)ldab);
    const i32x4_t rq = make_rsrc((const uint8_t*)p.qw + n0 * p.ldq * 4);
    const i32x4_t rs = make_rsrc((const uint8_t*)p.scales + n0 * p.lds * 2);

    // ---- A copies: wave quarter q fills rows 16q .. 16q+15 of the stage,
    // RPI rows per instruction; lane i lands at physical chunk i % 16 of its
    // row r, which holds logical chunk (i % 16) ^ (r % 16)
    uint32_t va[AI];
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const uint32_t r = wq * (BM / 4) + RPI * j + lane / CH;
        const uint32_t lc = (lane % CH) ^ (r % CH);
        va[j] = (int32_t)r < rows_a ? (wq * (BM / 4) + lane / CH) * ldab + lc * 16u : kOutOfRange;
    }
    // ---- word copies: instruction q of wave quarter w, lane i serves column
    // c = 16q + i/4 of the quarter and lands at byte 64c + 16(i % 4) of the
    // quarter's 2 KB, holding the column's 16-byte chunk (i % 4) ^ wsw(c).
    // The swizzle wsw(c) = (c / 4) % 4 spreads the 16 columns that one pass
    // of a 16-byte LDS read serves over all 64 banks (unswizzled, the 64-byte
    // column stride put four columns on each bank group).
    auto wsw = [](uint32_t c) __attribute__((always_inline)) -> uint32_t { return (c >> 2) & 3u; };
    uint32_t vq[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint32_t cq = 16u * q + lane / 4u, c = wq * 32u + cq;
        vq[q] = (int32_t)c < cols_b ? c * (uint32_t)(p.ldq * 4) + ((lane % 4u) ^ wsw(cq)) * 16u : kOutOfRange;
    }
    auto copy_step = [&](uint32_t kt) __attribute__((always_inline)) {
        const uint32_t slot = kt % NA;
        const uint32_t past = kt < KT ? 0u : kOutOfRange;  // past the last step: zeros, never used
#pragma unroll
        for (int j = 0; j < AI; ++j)
            load_lds_1k(ra, lds_a + slot * ASTAGE + (wq * (BM / 4) + RPI * j) * RB, va[j] | past,
                        kt * RB + (uint32_t)(RPI * j) * ldab);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            load_lds_1k(rq, lds_w + slot * WSTAGE + wq * 2048 + q * 1024, vq[q] | past, kt * 64u);
    };

    // ---- operands of a step: A fragments one sub-step ahead (two register
    // slots), this lane's 16 words and the step's scale
    const uint32_t lcol = lane & 31u, lhalf = lane >> 5;
    const uint32_t lsw = lcol % CH;
    Frag fa[4][TM];  // A fragments of sub-steps s .. s+2 in flight: slot s % 4
    u32x4 words[2];
    uint32_t scale;
    auto read_a = [&](uint32_t slot, int s, int fs) __attribute__((always_inline)) {
        const uint8_t* sa = lds_a + slot * ASTAGE;
        const uint32_t cs = (((8u * lhalf + (uint32_t)s) ^ lsw) << 4);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[fs][i] = lds128(sa, (i * 32 + lcol) * RB + cs);
    };
    // this lane's column's scales: row sc_row of lds_s, rotated by sc_rot pairs (see the prologue)
    const uint32_t half = G / 2;
    const uint32_t sc_col = wq * 32u + lcol, sc_row = sc_col * half * 4u, sc_rot = sc_col % half;
    auto read_b = [&](uint32_t kt, uint32_t slot) __attribute__((always_inline)) {
        const uint8_t* ws = lds_w + slot * WSTAGE + wq * 2048;
        words[0] = lds128(ws, lcol * 64u + (((2u * lhalf) ^ wsw(lcol)) << 4));
        words[1] = lds128(ws, lcol * 64u + (((2u * lhalf + 1u) ^ wsw(lcol)) << 4));
        // group kt is in pair kt/2, stored at (kt/2 + rot) mod half (in range
        // for the stale reads past the last step too: kt/2 <= half)
        uint32_t pr = kt / 2u + sc_rot;
        pr = pr >= half ? pr - half : pr;
        scale = *(const uint16_t*)(lds_s + sc_row + pr * 4u + (kt & 1u) * 2u);
    };
    const W4Consts wc = w4_consts(p.zero_point);
    auto dequant = [&](int s) __attribute__((always_inline)) {
        const _Float16 sc = bit_cast<_Float16>((uint16_t)scale);
        return dequant_w4_word(words[s >> 2][s & 3], wc, f16x2{sc, sc});
    };

    f32x16 acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
        acc[i] = f32x16{};
    auto mma = [&](const Frag& b, int fs) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            acc[i] = Mfma32<E_F16>::run(b, fa[fs][i], acc[i]);
    };

    // ---- prologue: every scale of the tile's columns (column c's G scales
    // in row c of lds_s, 2*G bytes, as G/2 four-byte pairs; instruction t of
    // the workgroup fills pair positions 64t .. 64t+63 of the flattened rows;
    // wave w issues t = w, w+8, ...), then each group's copies of its first
    // PER-1 steps.  Position p of row c holds pair (p - c) mod G/2: a step's
    // 32 lanes read one group of 32 consecutive columns, which this rotation
    // puts in 32 distinct banks (unrotated, a row stride of 2*G bytes put
    // them in two).
    {
        const uint32_t pairs = BN * half;
        for (uint32_t t = wave; t * 64u < pairs; t += 8u) {
            const uint32_t e = t * 64u + lane;
            const uint32_t c = e / half, pos = e - c * half;
            const uint32_t d = pos + half - c % half, dl = d >= half ? d - half : d;
            const uint32_t v = (e < pairs && (int32_t)c < cols_b) ? c * (uint32_t)(p.lds * 2) + dl * 4u : kOutOfRange;
            load_lds_256(rs, lds_s + t * 256u, v, 0u);
        }
    }
    copy_step(grp);
    copy_step(grp + 2u);
    wait_copies<CPS>();  // this wave's copies of its group's first step (and the scales) landed
    __syncthreads();     // ... and every wave's

    // ---- group steps.  Entering step kt, its words and scale and the A
    // fragments of its sub-steps 0 and 1 are in registers and the B operand
    // of sub-step 0 is dequantised.  Sub-step s issues its two MFMAs, the A
    // reads of sub-step s+2 and the dequant of sub-step s+1's word (VALU),
    // interleaved.  The barrier sits before the last sub-step, whose operands
    // are all in registers: past it the copies of the group's step kt+2 have
    // landed for every wave (published), and every read of step kt's slot is
    // done, so the slot is refilled with step kt+4 at once and the first
    // operands of step kt+2 are read while sub-step 7's MFMAs run.
    read_b(grp, grp % NA);
    read_a(grp % NA, 0, 0);
    read_a(grp % NA, 1, 1);
    Frag b = dequant(0);
    for (uint32_t kt = grp; kt < KT; kt += 2) {
        const uint32_t slot = kt % NA, nslot = (kt + 2) % NA;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < SUB - 1; ++s) {
            mma(b, s & 3);
            if (s + 2 < SUB)
                read_a(slot, s + 2, (s + 2) & 3);
            b = dequant(s + 1);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                if (s + 2 < SUB)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_copies<0>();  // this wave's copies of step kt+2 landed ...
        __syncthreads();   // ... and every wave's; every read of step kt is done
        __builtin_amdgcn_sched_barrier(0);
        copy_step(kt + 4);  // into the slot of step kt (zeros past the last step)
        // (past the group's last step these reads are stale and unused)
        read_b(kt + 2, nslot);
        read_a(nslot, 0, 0);
        read_a(nslot, 1, 1);
        mma(b, (SUB - 1) & 3);
        __builtin_amdgcn_sched_barrier(0);
        b = dequant(0);
    }
    wait_copies<0>();  // every copy (including those past the last step) has landed
    mfma_drain();

    // ---- sum the two groups' accumulators: group 1 leaves its blocks in
    // LDS (lane-contiguous 16-byte pieces), group 0 adds them
    constexpr int PBYTES = 4 * TM * 16 * 64 * 4;  // 4 waves x TM blocks x 16 floats x 64 lanes
    __syncthreads();
    uint8_t* part = lds_a + wq * (PBYTES / 4);
    if (grp == 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
                sts128(part, ((i * 4 + v4) * 64 + lane) * 16u,
                       bit_cast<u32x4>(f32x4{acc[i][4 * v4], acc[i][4 * v4 + 1], acc[i][4 * v4 + 2], acc[i][4 * v4 + 3]}));
    }
    __syncthreads();
    // ---- epilogue (fp16): group 0 adds group 1's partial blocks and stages
    // the whole BM x 128 tile in LDS (256-byte rows, 16-byte chunks XOR-
    // swizzled by row; wave quarter q writes chunks 4q .. 4q+3 of each row);
    // then all 8 waves store whole rows, 4 rows x 256 bytes per instruction
    // (partial-line stores cost far more).  Accumulator value v of lane l
    // holds row 32i + l%32, column 8*(v/4) + 4*(l/32) + v%4 of the wave's
    // 32 columns.
    constexpr int OB = BN * 2, NCH = OB / 16, TBYTES = BM * OB;
    static_assert(PBYTES + TBYTES <= NA * ASTAGE, "partials and staging must fit the A ring");
    uint8_t* ep = lds_a + PBYTES;
    if (grp == 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const f32x4 o = bit_cast<f32x4>(lds128(part, ((i * 4 + v4) * 64 + lane) * 16u));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i][4 * v4 + e] += o[e];
            }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint32_t r = i * 32 + lcol;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t c = wq * 4u + (uint32_t)g;  // 16-byte chunk of the tile row
                const uint32_t lo = (uint32_t)f32_to_f16_rne(acc[i][4 * g]) |
                                    ((uint32_t)f32_to_f16_rne(acc[i][4 * g + 1]) << 16);
                const uint32_t hi = (uint32_t)f32_to_f16_rne(acc[i][4 * g + 2]) |
                                    ((uint32_t)f32_to_f16_rne(acc[i][4 * g + 3]) << 16);
                *(u32x2*)(ep + r * OB + ((c ^ (r % NCH)) << 4) + lhalf * 8) = u32x2{lo, hi};
            }
        }
    }
    __syncthreads();  // the tile is staged
    uint16_t* C = (uint16_t*)p.C;
#pragma unroll
    for (int t = 0; t < BM * NCH / kW4Threads; ++t) {
        const uint32_t idx = t * kW4Threads + tid;
        const uint32_t r = idx / NCH, c = idx % NCH;
        const u32x4 q = lds128(ep, r * OB + ((c ^ (r % NCH)) << 4));
        const int64_t row = m0 + r, col = n0 + c * 8;
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

// --------------------------------------------------------------------------
// w4a16 for M <= 16 rows (decode).  Streaming the int4 weights from HBM is
// the whole cost, so nothing is staged in LDS: each lane loads 16 bytes of
// its column's words per 128-K group -- four words, 32 consecutive k -- and
// dequantises each word with tg::dequant_w4_word straight into the B operand
// of a 16x16x32 MFMA (M padded to 16 rows, rows past M read as zeros).
//
// K order inside an MFMA: the four lane quarters h = 0..3 of a 16x16x32 MFMA
// each supply 8 k values.  MFMA j (0..3) of a group gives quarter h the k
// = 128g + 32h + 8j .. +7, i.e. word 4h + j of the group: each lane's four
// words are one aligned 16-byte chunk, and its A operands are the four
// 16-byte chunks of the same 32 k of its row.  A and B agree on every k, so
// the sum is the group's full dot product.
//
// The waves of a workgroup split the K groups and reduce their partial tiles
// through LDS (the intra-block split-K of the TileScale README's GEMM
// example, section "Example of GEMM"); each workgroup owns 16*NT columns.
// Groups are loaded UNR at a time, double-buffered: the loads of the next
// batch are in flight while this batch is dequantised and multiplied.
// --------------------------------------------------------------------------
template <int WAVES, int NT, int UNR>
__global__ __launch_bounds__(WAVES * 64) void skinny_w4(TileArgs p)
{
    __shared__ float red[WAVES][NT][4][64];

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar offsets
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * NT);
    const uint32_t row = lane & 15u, quarter = lane >> 4;
    const int64_t KG = K / 128;  // K is a multiple of 128
    const int64_t g0 = KG * wave / WAVES, g1 = KG * (wave + 1) / WAVES;
    // Buffer loads with a fixed per-lane offset and the group's offset in the
    // scalar operand; rows past M and columns past N read through an
    // out-of-range offset, which returns zeros (no branches around the loads).
    // The host guarantees every valid offset stays below 2^31.
    const auto ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.A, (short)0, kNumRecords, kBufferFlags);
    const auto rq = __builtin_amdgcn_make_buffer_rsrc((void*)(p.qw + n0 * p.ldq), (short)0, kNumRecords, kBufferFlags);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)(p.scales + n0 * p.lds), (short)0, kNumRecords, kBufferFlags);
    // this lane's 64 bytes of A in group g: k = 128g + 32*quarter .. +31
    const uint32_t va = (int64_t)row < M ? row * (uint32_t)p.lda * 2u + quarter * 64u : kOutOfRange;
    uint32_t vq[NT], vs[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const bool ok = n0 + 16 * t + row < N;
        vq[t] = ok ? (16u * t + row) * (uint32_t)p.ldq * 4u + quarter * 16u : kOutOfRange;
        vs[t] = ok ? (16u * t + row) * (uint32_t)p.lds * 2u : kOutOfRange;
    }
    const W4Consts wc = w4_consts(p.zero_point);

    // two accumulators per tile (even and odd MFMA of a group), so that
    // consecutive MFMAs never wait on each other's result
    f32x4 acc[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    // loads of UNR groups starting at g (A chunks, int4 words, scales);
    // groups at or past g1 read zeros through the out-of-range offset
    auto load = [&](u32x4 (&a)[UNR][4], u32x4 (&q)[UNR][NT], uint32_t (&sc)[UNR][NT], int64_t g)
                    __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int32_t gg = (int32_t)(g + u);
            const uint32_t past = g + u < g1 ? 0u : kOutOfRange;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                a[u][j] = bit_cast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(ra, (int)(va | past), gg * 256 + j * 16, 0));
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                q[u][t] = bit_cast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(rq, (int)(vq[t] | past), gg * 64, 0));
                sc[u][t] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(vs[t] | past), gg * 2, 0);
            }
        }
    };
    auto compute = [&](u32x4 (&a)[UNR][4], u32x4 (&q)[UNR][NT], uint32_t (&sc)[UNR][NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < UNR; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const _Float16 s = bit_cast<_Float16>((uint16_t)sc[u][t]);
                    acc[t][j & 1] = Mfma16<E_F16>::run(a[u][j], dequant_w4_word(q[u][t][j], wc, f16x2{s, s}), acc[t][j & 1]);
                }
    };

    // Batches of UNR groups in two register buffers, two batches per trip
    // and no branch inside: the loads of one buffer are in flight while the
    // other is dequantised and multiplied.  A batch wholly or partly past g1
    // holds zeros (its products add nothing).
    u32x4 a0[UNR][4], a1[UNR][4], q0[UNR][NT], q1[UNR][NT];
    uint32_t s0[UNR][NT], s1[UNR][NT];  // one scale per register: nothing to pack after the loads
    const int64_t nb = (g1 - g0 + UNR - 1) / UNR;
    load(a0, q0, s0, g0);
    for (int64_t b = 0; b < nb; b += 2) {
        load(a1, q1, s1, g0 + (b + 1) * UNR);
        __builtin_amdgcn_sched_barrier(0);  // these loads issue before the compute they hide behind
        compute(a0, q0, s0);
        __builtin_amdgcn_sched_barrier(0);
        load(a0, q0, s0, g0 + (b + 2) * UNR);
        __builtin_amdgcn_sched_barrier(0);
        compute(a1, q1, s1);
        __builtin_amdgcn_sched_barrier(0);
    }

    mfma_drain();
    // partial tiles of this wave: value v of lane l is row 4*(l/16) + v, column l%16
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[wave][t][v][lane] = acc[t][0][v] + acc[t][1][v];
    __syncthreads();
    if (wave < NT) {  // wave t sums tile t over the K split, in wave order
        const int t = (int)wave;
        const int64_t col = n0 + 16 * t + row;
        uint16_t* C = (uint16_t*)p.C;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float sum = red[0][t][v][lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w)
                sum += red[w][t][v][lane];
            const int64_t r = (int64_t)quarter * 4 + v;
            if (r < M && col < N)
                C[r * p.ldc + col] = convert_out<O_F16>(sum);
        }
    }
}

// --------------------------------------------------------------------------
// The decode kernel with every operand copied to LDS (w4a16, 16 rows per
// workgroup: batches of more rows run one workgroup per 16-row slice; K a
// multiple of 1024, scales 4-byte aligned with an even stride).  The cost of
// skinny_w4 is the texture-address work of its load instructions, not their
// bytes: each 64-lane load takes the same address-unit time whether its
// lanes fetch a 64-byte half line (the int4 words), a scattered 16 bytes of
// A per row, or nothing (rows past M).  Here one copy instruction fetches
// whole 128-byte lines -- 8 columns x 2 groups of int4 words, or 2 rows x 256
// k of A -- and A needs only AI = ceil(M/2) of them per stage.
//
// Each wave owns a ring of RING LDS slots; a slot holds one stage of two
// 128-K groups: 32 columns of int4 words (128 B each, 16-byte chunks XOR-
// swizzled by column), 2*AI rows of A (512 B each, chunks swizzled by row;
// lanes of rows past 2*AI read a zeroed 16-byte block instead) and the
// stage's 64 scales.  The copies of stage s+RING-1 are issued before stage s
// is computed, so RING-1 stages are in flight behind the compute; a wave
// waits only for its own copies (no barrier in the loop).  The K order
// inside each MFMA is that of skinny_w4 (a lane's four words and its A
// chunks cover the same 32 k).
// --------------------------------------------------------------------------
template <int AI, int NT> struct W4dLayout {
    static constexpr int COLS = 16 * NT;  // columns per workgroup
    static constexpr int QB = COLS * 128, AB = 2 * AI * 512, SB = 256;
    static constexpr int SLOT = QB + AB + SB;
};

// Largest K range per wave with PRE (one A row and the scales held for the
// whole range): K <= kW4PreMaxKW * waves.
constexpr int kW4PreMaxKW = 4096;

// PRE (one row, AI = 1, 16 columns): each wave copies its K range of the A
// row (K_w * 2 bytes, 1 KiB per instruction) and its columns' scales for
// that range (4 stages of 16 columns per 256-byte instruction) into LDS
// once, before the ring, which then carries only the int4 words.  Per
// stage the ring otherwise copies two A rows of 256 k and 256 bytes of
// scales for 64 bytes used: at N = K = 8192 a timing-only copy without
// those copies ran 11.5 against 13.3 us per flushed launch.
template <int AI, int WAVES, int RING, int NT = 2, bool PRE = false>
__global__ __launch_bounds__(WAVES * 64) void skinny_w4_lds(TileArgs p)
{
    typedef W4dLayout<AI, NT> L;
    constexpr int QB = L::QB, AB = L::AB, COLS = L::COLS;
    static_assert(!PRE || (AI == 1 && NT == 1), "PRE: one A row, 16 columns");
    constexpr int SLOT = PRE ? QB : L::SLOT;           // ring slot: words (and A rows and scales)
    constexpr int APRE = PRE ? kW4PreMaxKW * 2 : 0;    // PRE: the wave's A row
    constexpr int SPRE = PRE ? kW4PreMaxKW / 256 * COLS * 4 : 0;  // PRE: [stage][column] scale pairs
    constexpr int WBYTES = RING * SLOT + APRE + SPRE;  // per wave
    constexpr int PER = PRE ? 2 * NT : 2 * NT + AI + 1;  // copy instructions per stage: words (A rows, scales)
    constexpr int ZERO = WAVES * WBYTES;  // 16 zero bytes shared by every wave
    static_assert(ZERO + 16 <= 160 * 1024 && WAVES * NT * 4 * 64 * 4 <= ZERO, "LDS");
    static_assert(AI >= 1 && AI <= 8 && RING >= 2 && (RING - 1) * PER <= 63, "copy ring");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[ZERO + 16];

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t N = p.N, K = p.K;
    // Rows come in slices of 16 (one per workgroup): workgroup id -> (column
    // block, slice) so that the S slices of a column block have ids 8 apart,
    // i.e. run on one XCD at about the same time and share its L2's copy of
    // the block's weights.  With S = 1 this is the identity.
    const int64_t S = (p.M + 15) / 16;
    const int64_t grp8 = (int64_t)blockIdx.x / (8 * S), rem = (int64_t)blockIdx.x % (8 * S);
    const int64_t slice = rem / 8, cb = grp8 * 8 + rem % 8;
    const int64_t n0 = cb * COLS;
    if (n0 >= N)
        return;  // padding of the last group of eight column blocks (whole workgroup)
    const int64_t M = p.M - 16 * slice < 16 ? p.M - 16 * slice : 16;  // rows of this slice
    const int64_t KG = K / 128;  // a multiple of 2*WAVES: every wave gets whole stages
    const int64_t g0 = KG * wave / WAVES, nst = KG / (2 * WAVES);
    uint8_t* ring = lds + wave * WBYTES;
    uint8_t* const apre = ring + RING * SLOT;  // PRE: stage st's 256 k of the A row at apre + 512 st
    uint8_t* const spre = apre + APRE;         // PRE: column c's scale pair of stage st at spre + 4 (COLS st + c)
    if (tid == 0)
        *(u32x4*)(lds + ZERO) = u32x4{0u, 0u, 0u, 0u};

    const i32x4_t ra = make_rsrc(p.A + 16 * slice * p.lda * 2);
    const i32x4_t rq = make_rsrc(p.qw + n0 * p.ldq);
    const i32x4_t rs = make_rsrc(p.scales + n0 * p.lds);
    // copy lanes: words -- instruction i, column 8i + lane/8, physical chunk
    // lane%8 holding logical chunk (lane%8) ^ ((column/2)%8); A -- instruction
    // i, row 2i + lane/32, physical chunk lane%32 holding logical chunk
    // (lane%32) ^ row; scales -- lane l < 32 takes the two of column l
    uint32_t vq[2 * NT], va[AI];
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
        const uint32_t col = 8u * i + lane / 8u;
        const uint32_t chunk = (lane % 8u) ^ ((col >> 1) & 7u);
        vq[i] = n0 + col < N ? col * (uint32_t)p.ldq * 4u + chunk * 16u : kOutOfRange;
    }
#pragma unroll
    for (int i = 0; i < AI; ++i) {
        const uint32_t row = 2u * i + lane / 32u;
        const uint32_t chunk = (lane % 32u) ^ row;
        va[i] = (int64_t)row < M ? row * (uint32_t)p.lda * 2u + chunk * 16u : kOutOfRange;
    }
    const uint32_t vs = (lane < (uint32_t)COLS && n0 + lane < N) ? lane * (uint32_t)p.lds * 2u : kOutOfRange;

    // stage st of this wave (groups g0 + 2st, +1) into ring slot `slot`;
    // a stage past the last one reads zeros (out-of-range offsets)
    auto issue = [&](int64_t st, uint8_t* slot) __attribute__((always_inline)) {
        const uint32_t past = st < nst ? 0u : kOutOfRange;
        const uint32_t g = (uint32_t)(g0 + 2 * st);
#pragma unroll
        for (int i = 0; i < 2 * NT; ++i)
            load_lds_1k(rq, slot + i * 1024, vq[i] | past, g * 64u);
        if constexpr (!PRE) {
#pragma unroll
            for (int i = 0; i < AI; ++i)
                load_lds_1k(ra, slot + QB + i * 1024, va[i] | past, g * 256u);
            load_lds_256(rs, slot + QB + AB, vs | past, g * 2u);
        }
    };
    // PRE: the wave's A row (instruction i: k = 128 g0 + 512 i + 8 lane ..
    // +7) and scale pairs (instruction i: stage 4i + lane/16 of column
    // lane%16), lanes past the wave's range or past N reading zeros; issued
    // before the ring, so every wait for a stage also covers them
    auto preload = [&]() __attribute__((always_inline)) {
        const int64_t kend = (g0 + 2 * nst) * 128;  // end of the wave's K range
        for (int64_t i = 0; i < (nst + 1) / 2; ++i) {
            const int64_t k = g0 * 128 + 512 * i + 8 * (int64_t)lane;
            load_lds_1k(ra, apre + i * 1024, k < kend ? lane * 16u : kOutOfRange,
                        (uint32_t)(g0 * 256 + 1024 * i));
        }
        const uint32_t c = lane % 16u;
        for (int64_t i = 0; i < (nst + 3) / 4; ++i) {
            const int64_t st = 4 * i + lane / 16u;
            const bool ok = st < nst && n0 + c < N;
            load_lds_256(rs, spre + i * 256, ok ? c * (uint32_t)p.lds * 2u + (lane / 16u) * 4u : kOutOfRange,
                         (uint32_t)(g0 * 2 + 16 * i));
        }
    };

    const W4Consts wc = w4_consts(p.zero_point);
    f32x4 acc[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t c = lane & 15u, h = lane >> 4;  // MFMA lane: column (or row) c, quarter h
    const bool arow = c < (PRE ? 1u : 2u * AI);     // this lane's A row is held in LDS (else zeros)

    // One stage: every LDS read first (words, scales and A chunks of both
    // groups), so a wave pays the LDS latency once per stage instead of once
    // per MFMA; then the dequant and the MFMAs, in the same order as before.
    auto compute = [&](const uint8_t* slot, int64_t st) __attribute__((always_inline)) {
        u32x4 q[2][NT], a[2][4];
        _Float16 sc[2][NT];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t col = 16u * t + c;
                const uint32_t phys = (4u * u + h) ^ ((col >> 1) & 7u);
                q[u][t] = lds128(slot, col * 128u + phys * 16u);
                const uint8_t* sp = PRE ? spre + ((uint32_t)st * COLS + col) * 4u : slot + QB + AB + col * 4u;
                sc[u][t] = bit_cast<_Float16>(*(const uint16_t*)(sp + u * 2u));
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t phys = (16u * u + 4u * h + j) ^ c;
                // (PRE: row 0 only, unswizzled: c = 0 where it is read)
                const uint32_t arow_at = PRE ? (uint32_t)(apre - lds) + (uint32_t)st * 512u + phys * 16u
                                             : (uint32_t)(slot - lds) + QB + c * 512u + phys * 16u;
                a[u][j] = lds128(lds, arow ? arow_at : (uint32_t)ZERO);
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[t][j & 1] = Mfma16<E_F16>::run(a[u][j], dequant_w4_word(q[u][t][j], wc, f16x2{sc[u][t], sc[u][t]}),
                                                       acc[t][j & 1]);
    };

    __syncthreads();  // the zero block is written
    if (nst > 0) {
        if constexpr (PRE)
            preload();
#pragma unroll
        for (int r = 0; r < RING - 1; ++r)
            issue(r, ring + r * SLOT);
        uint32_t cur = 0;  // slot of stage st
        for (int64_t st = 0; st < nst; ++st) {
            const uint32_t nxt = cur >= 1 ? cur - 1 : RING - 1;  // slot of stage st+RING-1 == slot of st-1
            issue(st + RING - 1, ring + nxt * SLOT);
            wait_copies<(RING - 1) * PER>();  // this wave's copies of stage st (and all before them) have landed
            __builtin_amdgcn_sched_barrier(0);
            compute(ring + cur * SLOT, st);
            __builtin_amdgcn_sched_barrier(0);
            cur = cur + 1 == RING ? 0 : cur + 1;
        }
    }
    wait_copies<0>();  // the trailing zero stages land before LDS is reused
    mfma_drain();

    // partial tiles: value v of lane l is row 4*(l/16) + v, column l%16
    __syncthreads();
    float* red = (float*)lds;  // [wave][tile][v][lane]
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            red[((wave * NT + t) * 4 + v) * 64 + lane] = acc[t][0][v] + acc[t][1][v];
    __syncthreads();
    for (int t = (int)wave; t < NT; t += WAVES) {  // wave t sums tile t over the K split, in wave order
        const int64_t col = n0 + 16 * t + c;
        uint16_t* C = (uint16_t*)p.C + 16 * slice * p.ldc;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float sum = red[(t * 4 + v) * 64 + lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w)
                sum += red[((w * NT + t) * 4 + v) * 64 + lane];
            const int64_t r = (int64_t)h * 4 + v;
            if (r < M && col < N)
                C[r * p.ldc + col] = convert_out<O_F16>(sum);
        }
    }
}

}  // namespace tg
