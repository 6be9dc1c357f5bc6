// The w4a16 Dequant-GEMM: fp16 activations x int4 weights (packed 8 per
// int32 along K, one fp16 scale per 128 K per column, a scalar zero point),
// fp32 accumulation, fp16 output.  Dequant-GEMM is one of the target kernels
// of "TileScale 与 TileLang比较" (sections 设计目标、定位与适用场景 and
// 生态互操作、性能、局限与路线图); the tile dataflow is the single-GPU GEMM
// skeleton of the same page (section 核心抽象与编程模型对比).
//
// Built on the NT kernel's machinery (tg_gemm_nt.hpp): A is copied straight
// into an NA-deep LDS ring with an XOR swizzle and read into MFMA fragments,
// with the same operand swap and staged fp16 epilogue.  B never passes
// through a shared stage: each wave owns 32 columns of the tile, copies
// their int4 words into its own LDS slot (alongside A's copies, NA steps
// ahead), reads them back and dequantises each word with
// tg::dequant_w4_word -- the routine tg_dequant_w4 also runs -- directly
// into the MFMA operand registers, interleaved with the MFMAs.  Each weight
// is dequantised once per workgroup.
//
// Copies retire in issue order, so a wait for one forces all older ones.  All
// copies of step j+NA are issued right after the barrier of step j, and the
// one wait per step (before that barrier, for step j+1) leaves the copies of
// the NA-2 later steps in flight.
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
// Work split: the workgroup computes a BM x 128 tile; wave w owns columns
// 32w .. 32w+31 and all BM rows (BM/32 accumulators of 32 x 32), so each
// weight is dequantised by exactly one wave, straight into the MFMA operand.
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
template <int BM, int NA>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_w4(TileArgs p)
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
    constexpr int CPS = AI + 2;      // copy instructions per wave per step
    // at the barrier opening step j: the copies of step j+1 were issued in
    // step j+1-NA, those of steps j+2 .. j+NA-1 may still fly
    constexpr int WAIT_BAR = (NA - 2) * CPS;
    static_assert(BM % 64 == 0 && NA >= 2 && (NA & (NA - 1)) == 0 && (NA - 1) * CPS <= 63,
                  "tile / ring depth / copies in flight");
    typedef u32x4 Frag;

    __shared__ __attribute__((aligned(1024))) uint8_t lds_a[NA * ASTAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_w[NA * WSTAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_s[BN * kW4MaxGroups * 2];

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

    // ---- A copies: wave w fills rows 16w .. 16w+15 of the stage, RPI rows
    // per instruction; lane i lands at physical chunk i % 16 of its row r,
    // which holds logical chunk (i % 16) ^ (r % 16)
    uint32_t va[AI];
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const uint32_t r = wave * (BM / 4) + RPI * j + lane / CH;
        const uint32_t lc = (lane % CH) ^ (r % CH);
        va[j] = (int32_t)r < rows_a ? (wave * (BM / 4) + lane / CH) * ldab + lc * 16u : kOutOfRange;
    }
    // ---- word copies: instruction q of wave w, lane i fetches 16-byte chunk
    // i % 4 of the 64 bytes of column 32w + 16q + i/4, landing at byte
    // 64 * (16q + i/4) + 16 * (i % 4) of the wave's 2 KB
    uint32_t vq[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const uint32_t c = wave * 32u + 16u * q + lane / 4u;
        vq[q] = (int32_t)c < cols_b ? c * (uint32_t)(p.ldq * 4) + (lane % 4u) * 16u : kOutOfRange;
    }
    auto copy_step = [&](uint32_t kt, uint32_t slot) __attribute__((always_inline)) {
        const uint32_t past = kt < KT ? 0u : kOutOfRange;  // past the last step: zeros, never used
#pragma unroll
        for (int j = 0; j < AI; ++j)
            load_lds_1k(ra, lds_a + slot * ASTAGE + (wave * (BM / 4) + RPI * j) * RB, va[j] | past,
                        kt * RB + (uint32_t)(RPI * j) * ldab);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            load_lds_1k(rq, lds_w + slot * WSTAGE + wave * 2048 + q * 1024, vq[q] | past, kt * 64u);
    };

    // ---- operands, read one whole step ahead into one of two register sets
    const uint32_t lcol = lane & 31u, lhalf = lane >> 5;
    const uint32_t lsw = lcol % CH;
    Frag fa[2][SUB][TM];
    u32x4 words[2][2];
    uint32_t scale[2];
    auto read_a = [&](uint32_t slot, int set, int s) __attribute__((always_inline)) {
        const uint8_t* sa = lds_a + slot * ASTAGE;
        const uint32_t cs = (((8u * lhalf + (uint32_t)s) ^ lsw) << 4);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[set][s][i] = lds128(sa, (i * 32 + lcol) * RB + cs);
    };
    auto read_b = [&](uint32_t kt, uint32_t slot, int set) __attribute__((always_inline)) {
        const uint8_t* ws = lds_w + slot * WSTAGE + wave * 2048;
        words[set][0] = lds128(ws, lcol * 64u + lhalf * 32u);
        words[set][1] = lds128(ws, lcol * 64u + lhalf * 32u + 16u);
        const uint32_t g = kt < KT ? kt : 0u;  // (the step after the last reads any valid entry)
        scale[set] = *(const uint16_t*)(lds_s + ((wave * 32u + lcol) * G + g) * 2u);
    };
    const W4Consts wc = w4_consts(p.zero_point);
    auto dequant = [&](int set, int s) __attribute__((always_inline)) {
        const _Float16 sc = bit_cast<_Float16>((uint16_t)scale[set]);
        return dequant_w4_word(words[set][s >> 2][s & 3], wc, f16x2{sc, sc});
    };

    f32x16 acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
        acc[i] = f32x16{};
    auto mma = [&](const Frag& b, int set, int s) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            acc[i] = Mfma32<E_F16>::run(b, fa[set][s][i], acc[i]);
    };

    // ---- prologue: every scale of the tile's columns (column c's G scales
    // at lds_s + 2*G*c, fetched as G/2 four-byte pairs; instruction t of the
    // workgroup takes pairs 64t .. 64t+63 of the flattened column-major
    // array; wave w issues t = w, w+4, ...), then the copies of steps
    // 0 .. NA-1, then the operands of step 0
    {
        const uint32_t half = G / 2, pairs = BN * half;
        for (uint32_t t = wave; t * 64u < pairs; t += 4u) {
            const uint32_t e = t * 64u + lane;
            const uint32_t c = e / half, d = e - c * half;
            const uint32_t v = (e < pairs && (int32_t)c < cols_b) ? c * (uint32_t)(p.lds * 2) + d * 4u : kOutOfRange;
            load_lds_256(rs, lds_s + t * 256u, v, 0u);
        }
    }
#pragma unroll
    for (int i = 0; i < NA; ++i)
        copy_step((uint32_t)i, (uint32_t)i);
    wait_copies<(NA - 1) * CPS>();  // scales and step 0 landed (this wave's part)
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SUB; ++s)
        read_a(0, 0, s);
    read_b(0, 0, 0);

    Frag b = dequant(0, 0);

    // ---- one step, in a fixed order.  The barrier opens the step: every
    // wave's copies of step kt+1 have landed, and every read of step kt's
    // slot (issued during step kt-1) is done, so the slot is refilled right
    // away.  The MFMAs then run on registers only.  Each sub-step interleaves
    // its two MFMAs with the sixteen VALU instructions that dequantise the
    // next word (the wave issues in order, so VALU work placed between two
    // MFMAs runs while the first executes) and with the reads of step kt+1;
    // the last sub-step dequantises word 0 of step kt+1.
    auto step = [&](uint32_t kt, int cur) __attribute__((always_inline)) {
        const uint32_t slot = kt % NA, next = (kt + 1) % NA;
        const int nxt = cur ^ 1;
        wait_copies<WAIT_BAR>();  // this wave's copies of step kt+1 landed
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        copy_step(kt + NA, slot);
        read_b(kt + 1, next, nxt);  // (stale, unused, after the last step)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < SUB; ++s) {
            mma(b, cur, s);
            read_a(next, nxt, s);
            b = s + 1 < SUB ? dequant(cur, s + 1) : dequant(nxt, 0);
            // MFMA, 8 VALU, 1 LDS read, MFMA, 8 VALU, 1 LDS read
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    for (uint32_t kt = 0; kt < KT; kt += 2) {  // KT is even
        step(kt, 0);
        step(kt + 1, 1);
#pragma unroll
        for (int s = 0; s < SUB; ++s)
#pragma unroll
            for (int i = 0; i < TM; ++i)
                pin(fa[0][s][i]);
        pin(words[0][0]);
        pin(words[0][1]);
        pin(scale[0]);
        pin(b);
    }
    wait_copies<0>();  // every copy (including those past the last step) has landed
    mfma_drain();

    // ---- epilogue (fp16): each wave stages its BM x 32 sub-tile in LDS and
    // stores 16-byte row pieces.  Accumulator value v of lane l holds row
    // 32i + l%32, column 8*(v/4) + 4*(l/32) + v%4 of the wave's columns.
    constexpr int WR = BM, OB = 64, NCH = 4, WBYTES = WR * OB;
    static_assert(4 * WBYTES <= NA * ASTAGE, "epilogue staging must fit the A ring");
    const int64_t wrow0 = m0, wcol0 = n0 + wave * 32;
    __syncthreads();
    uint8_t* ep = lds_a + wave * WBYTES;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const uint32_t r = i * 32 + lcol;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t lo = (uint32_t)f32_to_f16_rne(acc[i][4 * g]) |
                                ((uint32_t)f32_to_f16_rne(acc[i][4 * g + 1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_f16_rne(acc[i][4 * g + 2]) |
                                ((uint32_t)f32_to_f16_rne(acc[i][4 * g + 3]) << 16);
            *(u32x2*)(ep + r * OB + (((uint32_t)g ^ (r % NCH)) << 4) + lhalf * 8) = u32x2{lo, hi};
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    uint16_t* C = (uint16_t*)p.C;
#pragma unroll
    for (int t = 0; t < WR * NCH / 64; ++t) {
        const uint32_t idx = t * 64 + lane;
        const uint32_t r = idx / NCH, c = idx % NCH;
        const u32x4 q = lds128(ep, r * OB + ((c ^ (r % NCH)) << 4));
        const int64_t row = wrow0 + r, col = wcol0 + c * 8;
        if (row < M) {
            if (col + 8 <= N) {
                *(u32x4*)(C + row * p.ldc + col) = q;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col + e < N)
                        C[row * p.ldc + col + e] = (uint16_t)(q[e >> 1] >> ((e & 1) * 16));
            }
        }
    }
}

}  // namespace tg
