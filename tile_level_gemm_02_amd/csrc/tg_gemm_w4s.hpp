// The w4a16 Dequant-GEMM with K split over workgroups (tg_gemm_w4a16_ex):
// 128 x 128 output tiles, so that each dequantised int4 word feeds four
// MFMAs (one per 32-row block of the tile) instead of the two of the 64-row
// tile kernel (gemm_w4 in tg_gemm_w4.hpp), whose dequant VALU work outlasts
// its MFMAs; with few output tiles (M = 256 against N = 8192: 128 tiles)
// the K range is split over S workgroups per tile to fill the chip, each
// storing an fp32 partial tile in a caller workspace, the last one to
// finish adding them in split order (the split of K of the TileScale
// README's GEMM example, section "Example of GEMM", across workgroups).
// Dequant-GEMM is a target kernel of "TileScale 与 TileLang比较" (sections
// 设计目标、定位与适用场景 and 生态互操作、性能、局限与路线图).
//
// Work split inside a workgroup, as in gemm_w4: 8 waves, two per SIMD;
// waves w and w+4 own columns 32(w%4) .. +31 and all BM rows, wave w takes
// the even K steps of the workgroup's range and wave w+4 the odd ones, each
// into its own accumulators, summed through LDS at the end.  Each weight of
// the range is dequantised once in the workgroup, by the wave that
// multiplies it, straight into the MFMA operand (tg::dequant_w4_word, the
// routine tg_dequant_w4 runs).
//
// A K step is 64 wide (half a scale group).  The LDS holds a ring of NA
// steps of A (BM rows of 128 bytes), a ring of two periods of int4 words
// (a period is 4 steps: each column's whole 128-byte line), and, loaded
// once, the scales of the workgroup's groups.  A 32x32x16 MFMA takes, in lane l, eight k of row/column l % 32:
// sub-step s (0..3) gives lane half h the k = 32h + 8s .. +7, i.e. int4 word
// 4h + s of the column's 8 words of the step and 16-byte chunk 4h + s of the
// A row's 128 bytes (A and B agree on every k).
#pragma once

#include "tg_gemm_nt.hpp"
#include "tg_gemm_w4.hpp"

namespace tg {

constexpr int kW4sThreads = 512;
constexpr int kW4sMaxGroups = 64;  // scale groups per workgroup held in LDS (K per split <= 8192)

template <int NA_> struct W4sLayout {
    static constexpr int BM = 128, BN = 128, NA = NA_;
    static constexpr int ASTAGE = BM * 128;   // A rows of one step
    static constexpr int WPERIOD = BN * 128;  // words of 4 steps: 128 columns x 128 bytes (whole lines)
    static constexpr int OFF_W = NA * ASTAGE, OFF_S = OFF_W + 2 * WPERIOD;
    static constexpr int OFF_FLAG = OFF_S + BN * kW4sMaxGroups * 2;
    static constexpr int BYTES = OFF_FLAG + 16;
};

template <int NA_>
__global__ __launch_bounds__(kW4sThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_w4s(TileArgs p)
{
    typedef W4sLayout<NA_> L;
    constexpr int BM = L::BM, BN = L::BN, NA = L::NA;
    constexpr int RB = 128;          // bytes of K per staged A row: 64 fp16
    constexpr int RPI = 8;           // A rows per copy instruction
    constexpr int SUB = 4;           // MFMA sub-steps per step
    constexpr int TM = BM / 32;      // 32-row accumulators per wave
    constexpr int AI = BM / 4 / RPI; // A copy instructions per wave per step
    constexpr int WI = 2;            // word copy instructions per wave per period (of 4 steps)
    constexpr int PBYTES = 4 * TM * 16 * 64 * 4;  // group 1's partial blocks (epilogue)
    constexpr int OB = BN * 2, NCH = OB / 16, TBYTES = BM * OB;
    static_assert(PBYTES + TBYTES <= L::OFF_FLAG, "epilogue staging must fit the stage buffers");
    static_assert(8 * WI * 8 == BN, "the 8 waves' word copies cover the tile's columns");
    constexpr int PF = NA / 2;       // A steps in the ring per wave group
    static_assert(NA % 2 == 0 && PF >= 2 && (PF - 1) * AI + WI <= 63, "copy ring");
    typedef u32x4 Frag;

    __shared__ __attribute__((aligned(1024))) uint8_t lds[L::BYTES];
    uint8_t* const lds_a = lds;
    uint8_t* const lds_w = lds + L::OFF_W;
    uint8_t* const lds_s = lds + L::OFF_S;

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t grp = wave >> 2, wq = wave & 3u;  // K-step parity; column quarter
    const int64_t M = p.M, N = p.N, K = p.K;
    const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
    const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
    const uint32_t S = p.splits > 1u ? p.splits : 1u;
    uint32_t tmi, tni, ks;
    tile_split_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, S, p.group_m, tmi, tni, ks);
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
    const uint32_t ldab = (uint32_t)(p.lda * 2);
    const int32_t rows_a = (int32_t)(M - m0 < BM ? M - m0 : BM);
    const int32_t cols_b = (int32_t)(N - n0 < BN ? N - n0 : BN);
    // this workgroup's scale groups [g0, g0 + GW) (an even count, from an
    // even first group: the host splits K in whole pairs of groups) and its
    // K steps [kt0, kt0 + NK).  Wave group g runs steps 2i + g for
    // iterations i = 0 .. NIT-1; iteration i covers scale group g0 + i.
    const uint32_t G = (uint32_t)(K / 128);
    const uint32_t g0 = G * ks / S / 2u * 2u, g1 = ks + 1u == S ? G : G * (ks + 1u) / S / 2u * 2u;
    const uint32_t GW = g1 - g0, NK = 2u * GW, NIT = GW, kt0 = 2u * g0;
    const i32x4_t ra = make_rsrc(p.A + m0 * (int64_t)ldab);
    const i32x4_t rq = make_rsrc((const uint8_t*)p.qw + n0 * p.ldq * 4);
    const i32x4_t rs = make_rsrc((const uint8_t*)p.scales + n0 * p.lds * 2);

    // ---- A copies: wave quarter q fills rows 32q .. 32q+31 of the stage, 8
    // rows per instruction; lane i lands at physical chunk i % 8 of its row
    // r, which holds logical chunk (i % 8) ^ sw8(r): 16 rows (or columns
    // below) at one logical chunk then cover all 64 banks (two 128-byte rows
    // per bank line)
    auto sw8 = [](uint32_t r) __attribute__((always_inline)) -> uint32_t { return (r >> 1) & 7u; };
    uint32_t va[AI];
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const uint32_t r = wq * (BM / 4) + RPI * j + lane / 8u;
        va[j] = (int32_t)r < rows_a ? (wq * (BM / 4) + lane / 8u) * ldab + (((lane % 8u) ^ sw8(r)) << 4) : kOutOfRange;
    }
    // A rows of the step wave group grp runs in iteration i, into ring slot (2i + grp) % NA
    auto copy_a = [&](uint32_t i) __attribute__((always_inline)) {
        const uint32_t r = 2u * i + grp, slot = r % NA, kt = kt0 + r;
        const uint32_t past = r < NK ? 0u : kOutOfRange;  // past the range: zeros, never used
#pragma unroll
        for (int j = 0; j < AI; ++j)
            load_lds_1k(ra, lds_a + slot * L::ASTAGE + (wq * (BM / 4) + RPI * j) * RB, va[j] | past,
                        kt * RB + (uint32_t)(RPI * j) * ldab);
    };
    // ---- word copies, a period (4 steps, 256 k: one whole 128-byte line per
    // column) at a time: instruction t = 2*wave + u (0..15) of a period
    // serves columns 8t .. 8t+7, lane i column 8t + i/8, landing at physical
    // chunk i % 8 of the column's 128 bytes and holding its logical chunk
    // (i % 8) ^ sw8(column) -- 8 columns x 128 bytes per instruction, the
    // whole lines a vector L1 fetches with the fewest requests.  Period j
    // goes into word slot j % 2.
    uint32_t vw[WI];
#pragma unroll
    for (int u = 0; u < WI; ++u) {
        const uint32_t c = 8u * (2u * wave + (uint32_t)u) + lane / 8u;
        vw[u] = (int32_t)c < cols_b ? c * (uint32_t)(p.ldq * 4) + (((lane % 8u) ^ sw8(c)) << 4) : kOutOfRange;
    }
    auto copy_w = [&](uint32_t j) __attribute__((always_inline)) {
        const uint32_t past = 4u * j < NK ? 0u : kOutOfRange;
#pragma unroll
        for (int u = 0; u < WI; ++u)
            load_lds_1k(rq, lds_w + (j % 2u) * L::WPERIOD + (2u * wave + (uint32_t)u) * 1024u, vw[u] | past,
                        (kt0 + 4u * j) * 32u);
    };

    // ---- operands of a step
    const uint32_t lcol = lane & 31u, lhalf = lane >> 5;
    const uint32_t lsw = sw8(lcol);  // the A swizzle of every row this lane reads (rows 32i + lcol)
    Frag fa[4][TM];  // A fragments of sub-steps s .. s+2 in flight: slot s % 4
    u32x4 words;
    uint32_t scale;
    auto read_a = [&](uint32_t slot, int s, int fs) __attribute__((always_inline)) {
        const uint8_t* sa = lds_a + slot * L::ASTAGE;
        const uint32_t cs = (((4u * lhalf + (uint32_t)s) ^ lsw) << 4);
#pragma unroll
        for (int i = 0; i < TM; ++i)
            fa[fs][i] = lds128(sa, (i * 32 + lcol) * RB + cs);
    };
    // this lane's column's scales: row sc_col of lds_s (GW/2 four-byte pairs),
    // pair d stored at position (d + sc_col) mod GW/2 (see the prologue)
    const uint32_t half = GW / 2u;
    const uint32_t sc_col = wq * 32u + lcol, sc_row = sc_col * half * 4u, sc_rot = half > 0u ? sc_col % half : 0u;
    const uint32_t wcol = sc_col * 128u, wsw = sw8(sc_col);
    // words and scale of the step group grp runs in iteration i: logical
    // chunk 2q + lane half of the column's period line, q = (2i + grp) % 4
    auto read_b = [&](uint32_t i) __attribute__((always_inline)) {
        const uint32_t q = (2u * i + grp) & 3u;
        words = lds128(lds_w + ((i / 2u) % 2u) * L::WPERIOD, wcol + (((2u * q + lhalf) ^ wsw) << 4));
        const uint32_t g = i < GW ? i : GW - 1u;  // (clamped for the stale reads past the range)
        uint32_t pr = g / 2u + sc_rot;
        pr = pr >= half ? pr - half : pr;
        scale = *(const uint16_t*)(lds_s + sc_row + pr * 4u + (g & 1u) * 2u);
    };
    const W4Consts wc = w4_consts(p.zero_point);
    auto dequant = [&](int s) __attribute__((always_inline)) {
        const _Float16 sc = bit_cast<_Float16>((uint16_t)scale);
        return dequant_w4_word(words[s], wc, f16x2{sc, sc});
    };

    f32x16 acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
        acc[i] = f32x16{};
    auto mma_one = [&](const Frag& b, int fs, int i) __attribute__((always_inline)) {
        acc[i] = Mfma32<E_F16>::run(b, fa[fs][i], acc[i]);
    };

    // ---- prologue: the scales of the workgroup's groups for the tile's
    // columns (row c of lds_s: GW/2 pairs, position p holding pair
    // (p - c) mod GW/2, so that a step's 32 lanes -- 32 consecutive columns
    // at one group -- read 32 distinct banks), then the A rows of each
    // group's first two iterations and the words of the first period
    if (GW > 0u) {
        const uint32_t pairs = BN * half;
        for (uint32_t t = wave; t * 64u < pairs; t += 8u) {
            const uint32_t e = t * 64u + lane;
            const uint32_t c = e / half, pos = e - c * half;
            const uint32_t d = pos + half - c % half, dl = d >= half ? d - half : d;
            const uint32_t v =
                (e < pairs && (int32_t)c < cols_b) ? c * (uint32_t)(p.lds * 2) + (g0 / 2u + dl) * 4u : kOutOfRange;
            load_lds_256(rs, lds_s + t * 256u, v, 0u);
        }
    }
    copy_a(0);
    copy_w(0);
#pragma unroll
    for (int i = 1; i < PF; ++i)
        copy_a(i);
    wait_copies<(PF - 1) * AI>();  // this wave's scales, iteration 0's A rows and period 0's words landed ...
    __syncthreads();               // ... and every wave's

    // ---- iterations (as in gemm_w4): entering iteration i, the words and
    // scale of its step and the A fragments of its sub-steps 0 and 1 are in
    // registers and the B operand of sub-step 0 is dequantised.  Sub-step s
    // issues its TM MFMAs, the A reads of sub-step s+2 and the dequant of
    // sub-step s+1's word, interleaved.  The barrier sits before the last
    // sub-step, whose operands are all in registers: past it the copies the
    // next iteration reads have landed for every wave and every read of
    // iteration i's A slot is done, so that slot is refilled with the A rows
    // of iteration i+PF and, on even i, the other word slot with period
    // i/2 + 1 (its last reads were in iteration i-1), the words first; then
    // the first operands of iteration i+1 are read while the last MFMAs run.
    // Copies retire in order: iteration i+1 needs the A rows issued in
    // iteration i+1-PF and, when it opens a period, the words issued in
    // iteration i-1 before that iteration's A rows, so the wave lets the
    // (PF-2) * AI copies issued after those through.
    Frag b_op = {};
    auto iteration = [&](uint32_t i, auto odd) __attribute__((always_inline)) {
        const uint32_t slot = (2u * i + grp) % NA, nslot = (2u * i + 2u + grp) % NA;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < SUB - 1; ++s) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
                mma_one(b_op, s & 3, t);
            if (s + 2 < SUB)
                read_a(slot, s + 2, (s + 2) & 3);
            b_op = dequant(s + 1);
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 16 / TM, 0);
                if (s + 2 < SUB)
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_copies<(PF - 2) * AI>();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!decltype(odd)::value)
            copy_w(i / 2u + 1u);
        copy_a(i + (uint32_t)PF);  // into the slot of iteration i (zeros past the range)
        // (past the last iteration these reads are stale and unused)
        read_b(i + 1u);
        read_a(nslot, 0, 0);
        read_a(nslot, 1, 1);
#pragma unroll
        for (int t = 0; t < TM; ++t)
            mma_one(b_op, (SUB - 1) & 3, t);
        __builtin_amdgcn_sched_barrier(0);
        b_op = dequant(0);
    };
    if (NIT > 0u) {
        read_b(0);
        read_a(grp % NA, 0, 0);
        read_a(grp % NA, 1, 1);
        b_op = dequant(0);
    }
    for (uint32_t i = 0; i < NIT; i += 2) {  // NIT is even
        iteration(i, std::false_type{});
        iteration(i + 1u, std::true_type{});
    }
    wait_copies<0>();  // every copy (including those past the range) has landed
    mfma_drain();

    // ---- sum the two groups' accumulators: group 1 leaves its blocks in
    // LDS (lane-contiguous 16-byte pieces), group 0 adds them
    __syncthreads();
    uint8_t* part = lds + wq * (PBYTES / 4);
    if (grp == 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
                sts128(part, ((i * 4 + v4) * 64 + lane) * 16u,
                       bit_cast<u32x4>(f32x4{acc[i][4 * v4], acc[i][4 * v4 + 1], acc[i][4 * v4 + 2], acc[i][4 * v4 + 3]}));
    }
    __syncthreads();
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
    }

    // ---- K split: group 0's waves store the workgroup's partial tile and
    // the workgroup counts in at the tile's counter; the last of the S
    // arrivals adds the S partials in split order and stores the tile
    if (S > 1u) {
        constexpr int SHARE = TM * 1024;  // floats of a wave's share
        const uint32_t tile = tmi * tiles_n + tni;
        float* const share0 = p.partials + ((size_t)tile * S * 4 + wq) * SHARE;  // split 0's slot
        auto slot = [&](uint32_t q) __attribute__((always_inline)) { return share0 + (size_t)q * 4 * SHARE; };
        if (grp == 0) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    splitk_store(slot(ks), i, g, lane,
                                 f32x4{acc[i][4 * g], acc[i][4 * g + 1], acc[i][4 * g + 2], acc[i][4 * g + 3]});
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial stores are done
        }
        __syncthreads();  // ... and every wave's
        uint32_t* flag = (uint32_t*)(lds + L::OFF_FLAG);
        if (tid == 0) {
            const uint32_t old = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (old == S - 1u)  // every partial of the tile has arrived: the counter is free again
                __hip_atomic_exchange(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            *flag = old == S - 1u ? 1u : 0u;
        }
        __syncthreads();
        if (*flag == 0u)
            return;  // (uniform over the workgroup)
        asm volatile("" ::: "memory");  // no load of a partial is moved above the count
        if (grp == 0) {
            // acc = p_0 + p_1 + ... in split order; this workgroup's own share
            // p_ks is the accumulator itself (the bits it stored), only the
            // others are loaded (all of a partial's loads go out before its
            // adds: one wait per partial)
            f32x4 own[TM][4];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    own[i][g] = f32x4{acc[i][4 * g], acc[i][4 * g + 1], acc[i][4 * g + 2], acc[i][4 * g + 3]};
            for (uint32_t q = 0; q < S; ++q) {
                f32x4 v[TM][4];
                if (q != ks) {
                    const float* src = slot(q);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            v[i][g] = splitk_load(src, i, g, lane);
                } else {
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            v[i][g] = own[i][g];
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[i][4 * g + e] = q == 0u ? v[i][g][e] : acc[i][4 * g + e] + v[i][g][e];
            }
        }
    }

    // ---- epilogue (fp16): group 0 stages the whole BM x 128 tile in LDS
    // (256-byte rows, 16-byte chunks XOR-swizzled by row; wave quarter q
    // writes chunks 4q .. 4q+3 of each row); then all 8 waves store whole
    // rows.  Accumulator value v of lane l holds row 32i + l%32, column
    // 8*(v/4) + 4*(l/32) + v%4 of the wave's 32 columns.
    uint8_t* ep = lds + PBYTES;
    if (grp == 0) {
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
    for (int t = 0; t < BM * NCH / kW4sThreads; ++t) {
        const uint32_t idx = t * kW4sThreads + tid;
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

}  // namespace tg
