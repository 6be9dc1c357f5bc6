// 2:4 structured-sparse GEMM: C = A . W^T with A bf16 M x K (row-major) and
// W bf16 N x K holding at most 2 nonzeros in every aligned group of 4
// consecutive k, stored compressed (the kept values, [N][K/2], and a 4-bit
// code i0 | i1 << 2 of their positions per group, two per byte, [N][K/8]).
// The operation is the sparse GEMM T.gemm_sp in the TileLang timeline of
// "TileScale 与 TileLang比较"; the tile dataflow is the page's single-GPU GEMM
// skeleton (section 核心抽象与编程模型对比), as in the dense NT kernel.
//
// gfx950's sparse matrix instruction v_smfmac_f32_32x32x32_bf16 takes the
// compressed operand directly: for a 32 x 32 (dense) k block, lane l supplies
// row l%32 of the sparse operand as 8 kept values -- the groups 4h .. 4h+3
// of the block, h = l/32 -- and 16 bits of index, 2 per value, which is this
// format's codes for those 4 groups byte for byte.  The dense operand's lane l
// holds column l%32 at k = 8h .. 8h+7 and 16+8h .. 16+8h+7.  The weights are
// the sparse operand, so the output block is transposed exactly as in the
// NT kernel (lane l holds 4-column runs of output row l%32).
//
// Tile 256 x 256, 8 waves (2 x 4, each 128 x 64), a K step of 64: per step
// 32 KB of A rows (128 B per row, 16-byte chunks XOR-swizzled by row pair),
// 16 KB of kept values (64 B per row, chunks swizzled by row quad) and 2 KB
// of codes (8 B per row), all copied straight into LDS.  A ring of 3 such
// stages with one barrier per step: the copies of step k+3 are issued, spread
// between the MFMAs, right after the barrier that frees step k's stage.
//
// The copies bound this kernel (a step moves ≈50 KB into the compute unit
// for 1056 cycles of sparse MFMAs), and each copy instruction costs the
// address unit about the same whether it moves 1 KiB or the 256 bytes of a
// step's codes.  So with CP4 (K a multiple of 128) the codes are copied once
// per 4 steps, 16 bytes per lane (a row's codes of two steps), into a ring of
// two 8 KiB periods outside the stages: 25 copy instructions per wave per 4
// steps instead of 28.  Period layout: wave w's copy holds rows 32w .. 32w+31
// as [step pair][row][16 bytes], so a fragment read (32 consecutive rows of
// one step) touches 32 different banks.
#pragma once

#include "tg_gemm_nt.hpp"

namespace tg {

typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));

struct SpArgs {
    int64_t M, N, K;
    const uint8_t* A;
    int64_t lda;  // elements
    const uint8_t* Wv;
    int64_t ldv;  // elements
    const uint8_t* Wm;
    int64_t ldm;  // bytes
    void* C;
    int64_t ldc;  // elements
    uint32_t group_m;
};

// One wave instruction: 64 lanes x 4 bytes from global memory straight into
// the 256 bytes of LDS at address `dst` (lane i lands at dst + 4*i).
__device__ __forceinline__ void load_lds_256_at(i32x4_t r, uint32_t dst, uint32_t voff, uint32_t soff)
{
    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(r), "s"(soff), "{m0}"(dst)
                 : "memory");
}

// Waves per workgroup: 8 (2 x 4, each 128 x 64) or 4 (2 x 2, each 128 x 128).
// The copies are laid out for 8 copy slots of 32 rows each; with 4 waves each
// wave issues the copies of two slots.
template <int O, bool CP4, int NW = 8>
__global__ __launch_bounds__(64 * NW) void gemm_sp24(SpArgs p)
{
    static_assert(NW == 8 || NW == 4, "8 or 4 waves");
    constexpr int BM = 256, BN = 256, WM = 2, WN = NW / 2;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // 4 x 2 (8 waves) or 4 x 4 blocks of 32 x 32 per wave
    constexpr int VPW = 8 / NW;                          // copy slots per wave
    constexpr int KE = 64;                              // dense k per step
    constexpr int AB = BM * 128, VB = BN * 64, MB = CP4 ? 0 : BN * 8;
    constexpr int STAGE = AB + VB + MB;
    constexpr int NS = 3;
    constexpr int CPB = BN * 32;               // codes of a 4-step period (CP4)
    constexpr int CODES = NS * STAGE;          // offset of the two code periods (CP4)
    constexpr int BYTES = NS * STAGE + (CP4 ? 2 * CPB : 0);
    constexpr int PER = 4 + 2 + 1;  // copy instructions per slot per step: A rows, values, codes
    static_assert(BYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[BYTES];

    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t M = p.M, N = p.N, K = p.K;
    const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
    const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
    uint32_t tmi, tni;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, p.group_m, tmi, tni);
    const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
    const uint32_t ldab = (uint32_t)(p.lda * 2), ldvb = (uint32_t)(p.ldv * 2), ldmb = (uint32_t)p.ldm;
    const int32_t rows_a = (int32_t)(M - m0 < BM ? M - m0 : BM);
    const int32_t rows_w = (int32_t)(N - n0 < BN ? N - n0 : BN);
    const i32x4_t ra = make_rsrc(p.A + m0 * (int64_t)ldab);
    const i32x4_t rv = make_rsrc(p.Wv + n0 * (int64_t)ldvb);
    const i32x4_t rm = make_rsrc(p.Wm + n0 * (int64_t)ldmb);
    const int64_t KT = K / KE;  // K is a multiple of KE
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));

    // ---- copy lanes (copy slot w = VPW * wave + v; the slot's row offset
    // 32v joins the scalar offset).  A: instruction j covers rows 32w + 8j .. +7 (lane/8),
    // physical chunk lane%8 holding logical chunk (lane%8) ^ ((row/2)%8): one
    // value for even j, one for odd j.  Values: instruction j covers rows
    // 32w + 16j .. +15 (lane/4), physical chunk lane%4 holding logical chunk
    // (lane%4) ^ ((row/4)%4).  Codes: rows 32w .. +31 (lane/2), dword lane%2.
    const uint32_t slot0 = wave * VPW;  // first copy slot of this wave
    const uint32_t arow = slot0 * 32u + lane / 8u;
    const uint32_t ach0 = (lane % 8u) ^ ((lane / 16u) % 8u);
    const uint32_t ach1 = (lane % 8u) ^ ((4u + lane / 16u) % 8u);
    const uint32_t vrow = slot0 * 32u + lane / 4u;
    const uint32_t vch = (lane % 4u) ^ ((lane / 16u) % 4u);
    const uint32_t mrow = slot0 * 32u + lane / 2u;
    const uint32_t va0 = arow * ldab + ach0 * 16u, va1 = arow * ldab + ach1 * 16u;
    const uint32_t vv = vrow * ldvb + vch * 16u;
    const uint32_t vm = mrow * ldmb + (lane % 2u) * 4u;
    // CP4: lane l copies the codes of row 32w + l%32 for step pair l/32 of a period
    const uint32_t crow = slot0 * 32u + lane % 32u, cpair = lane / 32u;
    const uint32_t vc = crow * ldmb + cpair * 16u;

    // copy instruction qs (0 .. VPW*PER-1) of step kt into the stage at byte
    // offset `so`: instruction q = qs % PER of copy slot slot0 + qs / PER
    auto copy = [&](auto edge, int64_t kt, uint32_t so, int qs) __attribute__((always_inline)) {
        const int sv = qs / PER, q = qs % PER;
        const uint32_t sw32 = (uint32_t)sv * 32u;  // row offset of the slot past slot0
        const uint32_t sl = slot0 + (uint32_t)sv;   // the copy slot
        const uint32_t past = kt < KT ? 0u : kOutOfRange;
        const uint32_t base = lds0 + so;
        if (q < 4) {
            uint32_t v = ((q & 1) ? va1 : va0) | past;
            if constexpr (decltype(edge)::value)
                v |= (int32_t)(arow + sw32 + 8u * q) < rows_a ? 0u : kOutOfRange;
            load_lds_1k_at(ra, base + sl * 4096u + q * 1024u, v,
                           (uint32_t)kt * 128u + (uint32_t)(8 * q) * ldab + sw32 * ldab);
        } else if (q < 6) {
            const int j = q - 4;
            uint32_t v = vv | past;
            if constexpr (decltype(edge)::value)
                v |= (int32_t)(vrow + sw32 + 16u * j) < rows_w ? 0u : kOutOfRange;
            load_lds_1k_at(rv, base + AB + sl * 2048u + j * 1024u, v,
                           (uint32_t)kt * 64u + (uint32_t)(16 * j) * ldvb + sw32 * ldvb);
        } else if constexpr (!CP4) {
            uint32_t v = vm | past;
            if constexpr (decltype(edge)::value)
                v |= (int32_t)(mrow + sw32) < rows_w ? 0u : kOutOfRange;
            load_lds_256_at(rm, base + AB + VB + sl * 256u, v, (uint32_t)kt * 8u + sw32 * ldmb);
        } else if ((kt & 3) == 0) {  // CP4: the codes of steps kt .. kt+3 (pairs past K read zeros)
            uint32_t v = vc | (kt + 2 * (int64_t)cpair < KT ? 0u : kOutOfRange);
            if constexpr (decltype(edge)::value)
                v |= (int32_t)(crow + sw32) < rows_w ? 0u : kOutOfRange;
            load_lds_1k_at(rm, lds0 + CODES + (uint32_t)((kt >> 2) & 1) * CPB + sl * 1024u, v,
                           (uint32_t)kt * 8u + sw32 * ldmb);
        }
    };
    // copy instructions of this wave in the batch of step kt (the wait counts below)
    auto batch = [&](int64_t kt) __attribute__((always_inline)) { return VPW * (CP4 && (kt & 3) != 0 ? PER - 1 : PER); };

    // ---- fragments.  Every row a lane reads has the same swizzle.
    const uint32_t wm = wave / WN, wn = wave % WN;
    const uint32_t lrow = lane & 31u, h = lane >> 5;
    const uint32_t swa = (lrow / 2u) % 8u, swv = (lrow / 4u) % 4u;
    const uint32_t a_row0 = (wm * (BM / WM) + lrow) * 128u;
    const uint32_t w_row0 = wn * (BN / WN) + lrow;
    u32x4 fx[2][TM][2], fw[2][TN];
    uint32_t fi[2][TN];
    // fragment read r (0 .. TM+TN-1) of sub-step s of step kt (its stage at
    // byte offset `so`) into slot `slot`, numbered in the order the MFMAs
    // consume them: A block 0, every W block (values and codes), A blocks
    // 1 .. TM-1
    auto read_frag = [&](uint32_t so, int64_t kt, int s, int slot, int r) __attribute__((always_inline)) {
        const uint8_t* st = lds + so;
        if (r >= 1 && r <= TN) {
            const int j = r - 1;
            const uint32_t row = w_row0 + j * 32;
            fw[slot][j] = lds128(st, AB + row * 64u + ((((uint32_t)(2 * s) + h) ^ swv) << 4));
            if constexpr (CP4) {
                const uint32_t t = (uint32_t)kt & 3u;
                const uint32_t off = CODES + (uint32_t)((kt >> 2) & 1) * CPB + (row / 32u) * 1024u + (t >> 1) * 512u +
                                     (row % 32u) * 16u + (t & 1u) * 8u;
                fi[slot][j] = *(const uint16_t*)(lds + off + 4u * s + 2u * h);
            } else {
                fi[slot][j] = *(const uint16_t*)(st + AB + VB + row * 8u + 4u * s + 2u * h);
            }
        } else {
            const int i = r == 0 ? 0 : r - TN;
            const uint32_t row = a_row0 + i * 32 * 128;
            fx[slot][i][0] = lds128(st, row + ((((uint32_t)(4 * s) + h) ^ swa) << 4));
            fx[slot][i][1] = lds128(st, row + ((((uint32_t)(4 * s + 2) + h) ^ swa) << 4));
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{};
    // One sub-step (32 dense k): the TM*TN sparse MFMAs of fragment slot
    // `slot`.  The fragment reads of the next sub-step and NQ copy
    // instructions are spread evenly over them, each pinned in place, so the
    // in-order issue never waits on a burst.
    constexpr int NT = TM * TN, NR = TM + TN;
    auto substep = [&](int slot, auto rd, auto cp, auto nq) __attribute__((always_inline)) {
        constexpr int NQ = decltype(nq)::value;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int i = t / TN, j = t % TN;
            const u32x4 x0 = fx[slot][i][0], x1 = fx[slot][i][1];
            const i32x8 xb = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                              (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
            acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(bit_cast<bf16x8>(fw[slot][j]), bit_cast<bf16x16>(xb),
                                                                 acc[i][j], (int)fi[slot][j], 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (r * NT / NR == t)
                    rd(r);
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (q * NT / NQ == t)
                    cp(q);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto nothing = [](int) {};

    // One K step (2 sub-steps) on the stage at byte offset `cur` (step kt+1's
    // at `nxt`).  Entering, the fragments of its sub-step 0 are in slot 0.
    // The barrier publishes step kt+1 (step kt+2 may still be in flight) and
    // frees step kt's stage, into which step kt+3 is copied during the second
    // sub-step while step kt+1's first fragments are read.
    auto step = [&](auto edge, int64_t kt, uint32_t cur, uint32_t nxt) __attribute__((always_inline)) {
        substep(0, [&](int r) __attribute__((always_inline)) { read_frag(cur, kt, 1, 1, r); }, nothing,
                std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_barrier(0);
        if (batch(kt + 2) == VPW * PER)  // step kt+1 landed (step kt+2 may be in flight)
            wait_copies<VPW * PER>();
        else
            wait_copies<VPW * (PER - 1)>();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        // (the reads of step kt+1 after the last step are stale and unused)
        substep(1, [&](int r) __attribute__((always_inline)) { read_frag(nxt, kt + 1, 0, 0, r); },
                [&](int q) __attribute__((always_inline)) { copy(edge, kt + NS, cur, q); },
                std::integral_constant<int, VPW * PER>{});
    };
    auto run = [&](auto edge) __attribute__((always_inline)) {
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
            for (int q = 0; q < VPW * PER; ++q)
                copy(edge, st, (uint32_t)(st * STAGE), q);
        static_assert(NS == 3, "the prologue wait counts steps 1 and 2");
        wait_copies<VPW * (CP4 ? 2 * (PER - 1) : 2 * PER)>();  // step 0 landed (steps 1, 2 may be in flight)
        __syncthreads();
#pragma unroll
        for (int r = 0; r < NR; ++r)
            read_frag(0, 0, 0, 0, r);
        uint32_t cur = 0;  // byte offset of step kt's stage
        for (int64_t kt = 0; kt < KT; ++kt) {
            const uint32_t nxt = cur == (NS - 1) * STAGE ? 0u : cur + STAGE;
            step(edge, kt, cur, nxt);
            cur = nxt;
        }
        wait_copies<0>();  // copies past the last step (zeros) land before LDS is reused
    };
    if (KT > 0) {
        if (rows_a == BM && rows_w == BN)
            run(std::false_type{});
        else
            run(std::true_type{});
    }
    mfma_drain();

    // ---- epilogue (the NT kernel's layout: value v of lane l of acc[i][j] is
    // C[m = i*32 + l%32][n = j*32 + 8*(v/4) + 4*(l/32) + v%4] of the wave's sub-tile)
    constexpr int WR = BM / WM, WC = BN / WN;
    const int64_t wrow0 = m0 + wm * WR, wcol0 = n0 + wn * WC;
    if constexpr (O == O_F32) {
        // fp32 output: staged through LDS in passes of PR rows, stored as
        // whole rows (as the NT kernel does: a lane's 4 columns stored
        // directly make each store instruction write 32 rows x 32 bytes)
        constexpr int OB = WC * 4, NCH = OB / 16, PBY = NS * STAGE / NW;
        constexpr int PR = PBY / OB >= WR ? WR : (PBY / OB >= WR / 2 ? WR / 2 : WR / 4);
        static_assert(PR % 32 == 0 && WR % PR == 0 && (PR * NCH) % 64 == 0, "fp32 staging passes");
        __syncthreads();  // every wave is done reading the stages
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
                        const uint32_t c = (uint32_t)(8 * j + 2 * g) + h;  // columns j*32 + 8g + 4h .. +3
                        const f32x4 q = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
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
        // (row-major, 16-byte chunks XOR-swizzled by row), then writes whole rows
        constexpr int OB = WC * 2, NCH = OB / 16, WBYTES = WR * OB;
        static_assert(NW * WBYTES <= NS * STAGE, "epilogue staging must fit the stages");
        __syncthreads();  // every wave is done reading the stages
        uint8_t* ep = lds + wave * WBYTES;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint32_t r = i * 32 + lrow;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t c = (uint32_t)(4 * j + g);
                    const uint32_t lo = (uint32_t)convert_out<O>(acc[i][j][4 * g]) |
                                        ((uint32_t)convert_out<O>(acc[i][j][4 * g + 1]) << 16);
                    const uint32_t hi = (uint32_t)convert_out<O>(acc[i][j][4 * g + 2]) |
                                        ((uint32_t)convert_out<O>(acc[i][j][4 * g + 3]) << 16);
                    *(u32x2*)(ep + r * OB + ((c ^ (r % NCH)) << 4) + h * 8) = u32x2{lo, hi};
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
