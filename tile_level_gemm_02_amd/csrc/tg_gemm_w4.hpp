// The w4a16 Dequant-GEMM: fp16 activations x int4 weights (packed 8 per
// int32 along K, one fp16 scale per 128 K per column, a scalar zero point),
// fp32 accumulation, fp16 output.  Dequant-GEMM is one of the target kernels
// of "TileScale 与 TileLang比较" (sections 设计目标、定位与适用场景 and
// 生态互操作、性能、局限与路线图); the tile dataflow is the single-GPU GEMM
// skeleton of the same page (section 核心抽象与编程模型对比).
//
// Built on the NT kernel's machinery (tg_gemm_nt.hpp): A is copied straight
// into LDS, the same swizzle, fragment pipeline, operand swap and staged fp16
// epilogue.  B differs: each step's int4 words and scales are also copied
// straight into LDS (an NA-deep ring, like A), and one step before use every
// thread dequantises one column x 32 K of them (four words) with
// tg::dequant_w4_word -- the routine tg_dequant_w4 also runs -- into a
// swizzled two-stage fp16 B ring.  Each B element is thus dequantised once
// per workgroup, not once per wave that reads it.
//
// Copies retire in issue order, so a wait for one forces all older ones.  All
// copies of step j+NA are issued right after the barrier of step j, and the
// one wait per step (before the dequantisation of step j+1) leaves the copies
// of the NA-2 later steps in flight: every copy has about NA-1.5 steps to land.
#pragma once

#include <utility>

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

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N-1>{})
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// K must be a multiple of 256 (whole scale pairs), scales 4-byte aligned with
// an even row stride.
template <int BM, int BN, int NA>
__global__ __launch_bounds__(kThreads) void gemm_w4(TileArgs p)
{
    constexpr int RB = 128;           // bytes of K per staged row: 64 fp16
    constexpr int KE = 64;            // K elements per step
    constexpr int CH = 8, RPI = 8, RSW = 2;
    constexpr int TM = BM / 64, TN = BN / 64;
    constexpr int AI = BM / 32;       // A copy instructions per wave per step
    constexpr int ASTAGE = BM * RB, BSTAGE = BN * RB;
    constexpr int WSTAGE = 4096 + 1024;  // int4 words of a step (128 columns x 32 B), then scales
    constexpr int CPS = AI + 2;          // copy instructions per wave per step
    // before the dequantisation of step j+1 in step j: its copies were issued
    // in step j+1-NA; those of steps j+2-NA .. j-1 may still be in flight
    constexpr int WAIT_DQ = (NA - 2) * CPS;
    static_assert(BN == 128 && BN * 2 == kThreads, "one (column, half-step) unit of B words per thread");
    static_assert(NA >= 2 && (NA - 1) * CPS <= 63, "copies in flight");
    typedef u32x4 Frag;

    __shared__ __attribute__((aligned(1024))) uint8_t lds_a[NA * ASTAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_w[NA * WSTAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_b[2 * BSTAGE];

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
    const int64_t KT = K / KE;
    const i32x4_t ra = make_rsrc(p.A + m0 * (int64_t)ldab);
    const i32x4_t rq = make_rsrc((const uint8_t*)p.qw + n0 * p.ldq * 4);
    const i32x4_t rs = make_rsrc((const uint8_t*)p.scales + n0 * p.lds * 2);

    // ---- A copies (as in the NT kernel: 128-byte rows, swizzle (row/2)%8)
    const uint32_t lrowi = lane / CH;
    const uint32_t lchunk0 = (lane % CH) ^ ((lrowi / RSW) % CH);
    const uint32_t lchunk1 = (lane % CH) ^ ((4u + lrowi / RSW) % CH);
    const uint32_t va0 = (wave * (BM / 4) + lrowi) * ldab + lchunk0 * 16u;
    const uint32_t va1 = (wave * (BM / 4) + lrowi) * ldab + lchunk1 * 16u;
    // ---- B copies: wave w fetches columns 32w .. 32w+31 of the tile: the 32
    // bytes of int4 words of one step per column (two lanes, 16 bytes each:
    // lane i takes column 32w + i/2, half i%2), and per column the 4-byte
    // pair of scales that covers the step (lanes 0..31; lanes 32..63 fetch
    // nothing and write zeros to an unused slot)
    const uint32_t qcol = wave * 32u + lane / 2u;
    const uint32_t vq = (int32_t)qcol < cols_b ? qcol * (uint32_t)(p.ldq * 4) + (lane & 1u) * 16u : kOutOfRange;
    const uint32_t scol = wave * 32u + (lane & 31u);
    const uint32_t vs = (lane < 32u && (int32_t)scol < cols_b) ? scol * (uint32_t)(p.lds * 2) : kOutOfRange;
    auto copy_step = [&](int64_t kt) __attribute__((always_inline)) {
        const uint32_t past = kt < KT ? 0u : kOutOfRange;  // past the last step: zeros, never used
        const uint32_t slot = (uint32_t)(kt % NA);
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            uint32_t v = ((j & 1) ? va1 : va0) | past;
            v |= (int32_t)(wave * (BM / 4) + RPI * j + lrowi) < rows_a ? 0u : kOutOfRange;
            load_lds_1k(ra, lds_a + slot * ASTAGE + wave * (BM / 4) * RB + j * 1024, v,
                        (uint32_t)kt * RB + (uint32_t)(RPI * j) * ldab);
        }
        uint8_t* ws = lds_w + slot * WSTAGE;
        load_lds_1k(rq, ws + wave * 1024, vq | past, (uint32_t)kt * 32u);
        load_lds_256(rs, ws + 4096 + wave * 256, vs | past, (uint32_t)(kt >> 2) * 4u);
    };

    // ---- dequantisation: thread t takes column t/2 of the tile, K offsets
    // 32*(t%2) .. +31 of the step (the 16 bytes its own lane fetched, so only
    // this wave's copy wait is needed), and writes them as fp16 into logical
    // chunks 4*(t%2) .. +3 of row t/2 of B stage kt % 2
    const uint32_t bcol = tid >> 1, bhalf = tid & 1u;
    const uint32_t bsw = (bcol / RSW) % CH;
    const W4Consts wc = w4_consts(p.zero_point);
    auto dequant_b = [&](int64_t kt) __attribute__((always_inline)) {
        const uint8_t* ws = lds_w + (uint32_t)(kt % NA) * WSTAGE;
        const u32x4 q = lds128(ws, tid * 16u);
        const uint32_t pair = *(const uint32_t*)(ws + 4096 + wave * 256 + (lane >> 1) * 4);
        const _Float16 s = bit_cast<_Float16>((uint16_t)(pair >> (((uint32_t)kt & 2u) << 3)));
        const f16x2 s2{s, s};
        uint8_t* row = lds_b + (uint32_t)(kt & 1) * BSTAGE + bcol * RB;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            sts128(row, ((bhalf * 4u + (uint32_t)w) ^ bsw) << 4, dequant_w4_word(q[w], wc, s2));
    };

    // ---- fragments
    const uint32_t wm = wave >> 1, wn = wave & 1u;
    const uint32_t lrow = lane & 31u, lgrp = lane >> 5;
    const uint32_t sw = (lrow / RSW) % CH;
    const uint32_t a_row0 = (wm * (BM / 2) + lrow) * RB;
    const uint32_t b_row0 = (wn * (BN / 2) + lrow) * RB;
    Frag fa[2][TM], fb[2][TN];
    auto read_frags = [&](int64_t kt, int s, int slot) __attribute__((always_inline)) {
        const uint8_t* sa = lds_a + (uint32_t)(kt % NA) * ASTAGE;
        const uint8_t* sb = lds_b + (uint32_t)(kt & 1) * BSTAGE;
        const uint32_t cs = ((((uint32_t)(2 * s) + lgrp) ^ sw) << 4);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[slot][i] = lds128(sa, a_row0 + i * 32 * RB + cs);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            fb[slot][j] = lds128(sb, b_row0 + j * 32 * RB + cs);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{};
    auto mma = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = Mfma32<E_F16>::run(fb[slot][j], fa[slot][i], acc[i][j]);
    };

    // ---- prologue: the copies of steps 0 .. NA-1
#pragma unroll
    for (int i = 0; i < NA; ++i)
        copy_step(i);
    wait_copies<(NA - 1) * CPS>();  // step 0 landed (this wave's part)
    dequant_b(0);
    __syncthreads();
    read_frags(0, 0, 0);

    // ---- main loop
    auto step = [&](int64_t kt) __attribute__((always_inline)) {
        read_frags(kt, 1, 1);
        mma(0);
        read_frags(kt, 2, 0);
        wait_copies<WAIT_DQ>();  // this wave's copies of step kt+1 landed (A, words, scales)
        dequant_b(kt + 1);       // into B stage (kt+1)%2, free since the last barrier
        mma(1);
        read_frags(kt, 3, 1);
        mma(0);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();  // A and B of step kt+1 complete for every wave; A stage kt%NA free
        __builtin_amdgcn_sched_barrier(0);
        copy_step(kt + NA);        // into slot kt % NA
        read_frags(kt + 1, 0, 0);  // (stale, unused, after the last step)
        mma(1);
    };
    for (int64_t kt = 0; kt < KT; kt += NA) {
        static_for<NA>([&](auto ic) __attribute__((always_inline)) {
            if (kt + decltype(ic)::value < KT)
                step(kt + decltype(ic)::value);
        });
    }
    wait_copies<0>();  // every copy (including those past the last step) has landed
    mfma_drain();

    // ---- epilogue (fp16): stage each wave's sub-tile in LDS, 16-byte row stores
    constexpr int WR = BM / 2, WC = BN / 2;
    constexpr int OB = WC * 2, NCH = OB / 16, WBYTES = WR * OB;
    static_assert(4 * WBYTES <= NA * ASTAGE, "epilogue staging must fit the A ring");
    const int64_t wrow0 = m0 + wm * WR, wcol0 = n0 + wn * WC;
    __syncthreads();
    uint8_t* ep = lds_a + wave * WBYTES;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const uint32_t r = i * 32 + lrow;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t c = (uint32_t)(4 * j + g);
                const uint32_t lo = (uint32_t)f32_to_f16_rne(acc[i][j][4 * g]) |
                                    ((uint32_t)f32_to_f16_rne(acc[i][j][4 * g + 1]) << 16);
                const uint32_t hi = (uint32_t)f32_to_f16_rne(acc[i][j][4 * g + 2]) |
                                    ((uint32_t)f32_to_f16_rne(acc[i][j][4 * g + 3]) << 16);
                *(u32x2*)(ep + r * OB + ((c ^ (r % NCH)) << 4) + lgrp * 8) = u32x2{lo, hi};
            }
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
