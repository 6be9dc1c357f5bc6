// Host-side helpers of the C ABI: argument validation and kernel launch.
// Validation runs before any HIP call, so a rejected call launches nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg.h"
#include "tg_gemm_nt.hpp"
#include "tg_gemm_skinny.hpp"
#include "tg_kernels.hpp"

namespace tg {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0u; }

inline int out_bytes(tg_dtype d) { return d == TG_F32 ? 4 : 2; }

// Validate a dense GEMM call (A: M x K, B: K x N in `b_layout`, C: M x N).
// Returns TG_OK and sets *empty when nothing is to be computed.
inline tg_status check_dense(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                             const void* B, int64_t ldb, int b_layout, void* C, int64_t ldc,
                             int c_dtype, int elem_bytes, bool* empty)
{
    *empty = false;
    if (M < 0 || N < 0 || K < 0)
        return TG_ERR_INVALID_VALUE;
    if (b_layout != TG_ROW_MAJOR && b_layout != TG_COL_MAJOR)
        return TG_ERR_INVALID_VALUE;
    if (c_dtype != TG_F32 && c_dtype != TG_F16 && c_dtype != TG_BF16)
        return TG_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) {
        *empty = true;
        return TG_OK;
    }
    if (C == nullptr || ldc < N)
        return TG_ERR_INVALID_VALUE;
    if (K > 0) {
        if (A == nullptr || B == nullptr)
            return TG_ERR_INVALID_VALUE;
        if (lda < K)
            return TG_ERR_INVALID_VALUE;
        if (ldb < (b_layout == TG_ROW_MAJOR ? N : K))
            return TG_ERR_INVALID_VALUE;
        if (!aligned16(A) || !aligned16(B) || ((lda * elem_bytes) & 15) || ((ldb * elem_bytes) & 15))
            return TG_ERR_MISALIGNED;
    }
    if (!aligned16(C) || ((ldc * out_bytes((tg_dtype)c_dtype)) & 15))
        return TG_ERR_MISALIGNED;
    return TG_OK;
}

inline tg_status launched()
{
    return hipGetLastError() == hipSuccess ? TG_OK : TG_ERR_LAUNCH;
}

template <int BM, int BN>
inline int64_t n_tiles(int64_t M, int64_t N)
{
    return ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
}

template <int E, int BL, int O, int BM, int BN, bool W4>
tg_status launch_tile(const TileArgs& a, hipStream_t s)
{
    const int64_t tiles = n_tiles<BM, BN>(a.M, a.N);
    if (tiles > 0x7FFFFFFF)
        return TG_ERR_NOT_SUPPORTED;
    hipLaunchKernelGGL((tile_gemm<E, BL, O, BM, BN, W4>), dim3((uint32_t)tiles), dim3(kThreads), 0, s, a);
    return launched();
}

// Tile edge for a dense problem: the largest tile that still gives enough
// workgroups to spread over the chip's 256 compute units.
inline int pick_tile(int64_t M, int64_t N, bool allow256)
{
    if (allow256 && n_tiles<256, 256>(M, N) >= 192)
        return 256;
    if (n_tiles<128, 128>(M, N) >= 96)
        return 128;
    return 64;
}

template <int E, int BL, int O>
tg_status launch_tile_sized(TileArgs& a, hipStream_t s)
{
    const int t = pick_tile(a.M, a.N, BL == B_KCONTIG);
    a.group_m = 4;
    if constexpr (BL == B_KCONTIG) {
        if (t == 256)
            return launch_tile<E, BL, O, 256, 256, false>(a, s);
    }
    if (t >= 128)
        return launch_tile<E, BL, O, 128, 128, false>(a, s);
    return launch_tile<E, BL, O, 64, 64, false>(a, s);
}

// The direct-to-LDS NT kernel needs whole 16-byte chunks along K and 32-bit
// buffer offsets over one tile (BM rows of A / BN rows of B plus one K span).
template <int E>
inline bool nt_eligible(const TileArgs& a)
{
    constexpr int EB = ElemInfo<E>::bytes;
    const int64_t lim = (int64_t)kNumRecords;
    return (a.K % (16 / EB)) == 0 && 256 * a.lda * EB + a.K * EB < lim && 256 * a.ldb * EB + a.K * EB < lim;
}

// The NT kernel with an N-contiguous (row-major) B: whole 16-byte chunks
// along K for A and along N for B, and 32-bit buffer offsets over the K rows
// of B (plus the rows of the steps past K that the ring forms).  8-bit B rows
// of a 64-wide tile would be 64 bytes, too narrow for its staging: fp8 takes
// this path only where the 128 or 256 tile is picked.
template <int E>
inline bool nt_eligible_nrow(const TileArgs& a)
{
    constexpr int EB = ElemInfo<E>::bytes, CE = 16 / EB, KE = 128 / EB;
    const int64_t lim = (int64_t)kNumRecords;
    if (EB == 1 && pick_tile(a.M, a.N, true) < 128)
        return false;
    return (a.K % CE) == 0 && (a.N % CE) == 0 && 256 * a.lda * EB + a.K * EB < lim &&
           (a.K + 6 * KE) * a.ldb * EB + 256 * EB < lim;
}

// Staging of the NT kernel: bytes of K per staged row, and LDS half-stages in
// the ring.  For 16-bit inputs four (two full stages) measured faster than
// five on the 256 x 256 tile at 4096^3 (the fifth fills the LDS: 5 x 32 KB);
// fp8 at 8192^3, whose copies miss L2 more often and wait longer, runs ~9%
// faster with the fifth.
template <int E> struct NtStaging { static constexpr int RB = 128; };
template <int E, int BM> struct NtRing { static constexpr int NH = 4; };
template <> struct NtRing<E_FP8, 256> { static constexpr int NH = 5; };

// Waves of the NT kernel per tile: the 256 x 256 tile takes 8 (2 x 4, two
// per SIMD) for the LDS read rate its fragments need; smaller tiles take 4.
template <int BM, int BN> struct NtWaves { static constexpr int WM = 2, WN = 2; };
template <> struct NtWaves<256, 256> { static constexpr int WM = 2, WN = 4; };

template <int E, int O, int BM, int BN, int BL = B_KCONTIG, int NH = NtRing<E, BM>::NH>
tg_status launch_nt(const TileArgs& a, hipStream_t s)
{
    const int64_t tiles = n_tiles<BM, BN>(a.M, a.N);
    if (tiles > 0x7FFFFFFF)
        return TG_ERR_NOT_SUPPORTED;
    constexpr int RB = NtStaging<E>::RB;
    constexpr int WM = NtWaves<BM, BN>::WM, WN = NtWaves<BM, BN>::WN;
    hipLaunchKernelGGL((gemm_nt<E, O, BM, BN, RB, NH, WM, WN, BL>), dim3((uint32_t)tiles), dim3(64 * WM * WN), 0, s, a);
    return launched();
}

// The 128 and 64 tiles: a ring of 8 half-stages (4 steps in flight) when the
// tiles fit the chip at the occupancy that allows (one 128 KiB workgroup, or
// two of 64 KiB, per CU); else 4, which leaves room for more resident
// workgroups.  A small tile does little MFMA work per K step, so with 2 steps
// in flight it waits on copy latency: at N = K = 8192, M = 128 (64 tiles)
// 96 -> 45 us, M = 256 (128 tiles) 114 -> 77 us; 2048^3 27 -> 21 us.
// (pick_tile takes the 64 tile only below 96 tiles of 128, i.e. for at
// most 384 tiles of 64: always the deep ring.)
template <int E, int O, int BM, int BL>
tg_status launch_nt_ring(const TileArgs& a, hipStream_t s)
{
    if constexpr (BM == 64) {
        return launch_nt<E, O, 64, 64, BL, 8>(a, s);
    } else {
        if (n_tiles<BM, BM>(a.M, a.N) <= 256)
            return launch_nt<E, O, BM, BM, BL, 8>(a, s);
        return launch_nt<E, O, BM, BM, BL, 4>(a, s);
    }
}

template <int E, int O, int BL = B_KCONTIG>
tg_status launch_nt_sized(TileArgs& a, hipStream_t s)
{
    a.group_m = 4;
    const int t = pick_tile(a.M, a.N, true);
    if (t == 256)
        return launch_nt<E, O, 256, 256, BL>(a, s);
    if constexpr (ElemInfo<E>::bytes == 1 && BL == B_NCONTIG)
        return launch_nt_ring<E, O, 128, BL>(a, s);  // (nt_eligible_nrow has ruled out the 64 tile)
    else if (t == 128)
        return launch_nt_ring<E, O, 128, BL>(a, s);
    else
        return launch_nt_ring<E, O, 64, BL>(a, s);
}

template <int E, int BL>
tg_status launch_dense(TileArgs& a, int c_dtype, hipStream_t s)
{
    if constexpr (BL == B_KCONTIG) {
        if (nt_eligible<E>(a)) {
            switch (c_dtype) {
            case TG_F32: return launch_nt_sized<E, O_F32>(a, s);
            case TG_F16: return launch_nt_sized<E, O_F16>(a, s);
            default: return launch_nt_sized<E, O_BF16>(a, s);
            }
        }
    } else {
        if (nt_eligible_nrow<E>(a)) {
            switch (c_dtype) {
            case TG_F32: return launch_nt_sized<E, O_F32, B_NCONTIG>(a, s);
            case TG_F16: return launch_nt_sized<E, O_F16, B_NCONTIG>(a, s);
            default: return launch_nt_sized<E, O_BF16, B_NCONTIG>(a, s);
            }
        }
    }
    switch (c_dtype) {
    case TG_F32: return launch_tile_sized<E, BL, O_F32>(a, s);
    case TG_F16: return launch_tile_sized<E, BL, O_F16>(a, s);
    default: return launch_tile_sized<E, BL, O_BF16>(a, s);
    }
}

// Launch shape of the skinny kernel: waves per workgroup (each streams its
// own K range) and LDS ring slots per wave.
struct SkinnyCfg {
    static constexpr int WAVES = 8, RING = 2;
};

// Workgroups per column block of the skinny kernel: two workgroups per CU
// (512) when N alone gives fewer, keeping at least two 64-wide K stages per
// wave.
inline int skinny_split(int64_t blocks, int64_t K)
{
    int64_t split = (512 + blocks - 1) / blocks;
    const int64_t most = K / kSkKE / (SkinnyCfg::WAVES * 2);
    if (split > most)
        split = most;
    return split > 1 ? (int)split : 1;
}

template <int E, int O, int AI, bool SPLIT>
void launch_skinny_ai(const SkinnyArgs& sa, int64_t blocks, int split, hipStream_t s)
{
    typedef SkinnyCfg G;
    hipLaunchKernelGGL((skinny_gemm<E, O, G::WAVES, AI, G::RING, SPLIT>), dim3((uint32_t)blocks, (uint32_t)split),
                       dim3(64 * G::WAVES), 0, s, sa);
}

// A rows are copied 8 at a time: one copy instruction for M <= 8, two above.
template <int E, int O, bool SPLIT = false>
void launch_skinny(const SkinnyArgs& sa, int64_t blocks, int split, hipStream_t s)
{
    if (sa.M <= 8)
        launch_skinny_ai<E, O, 1, SPLIT>(sa, blocks, split, s);
    else
        launch_skinny_ai<E, O, 2, SPLIT>(sa, blocks, split, s);
}

// Batches up to this many rows against a K-contiguous B take the skinny
// kernel, in 16-row slices (each slice re-reads B, mostly from L2).  At
// N = K = 8192 (bf16, flushed): 17 rows 37 us and 32 rows 43 against 46 for
// the 64-tile NT kernel; from 40 rows on (53 us) the tile kernel is faster.
constexpr int64_t kSkSliceMaxM = 32;

// fp16 / bf16 GEMM.  Few rows (kSkSliceMaxM) against a K-contiguous B take
// the skinny kernel; everything else the tile kernel (K == 0 runs it with no
// K steps, which stores zeros: the empty sum).
template <int E>
tg_status gemm_16bit(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, int b_layout, void* C, int64_t ldc, int c_dtype, void* stream)
{
    bool empty;
    tg_status st = check_dense(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, 2, &empty);
    if (st != TG_OK || empty)
        return st;
    hipStream_t s = (hipStream_t)stream;
    typedef SkinnyCfg G;
    if (M <= kSkSliceMaxM && b_layout == TG_COL_MAJOR && K > 0 && skinny_offsets_fit(K, lda, ldb, G::RING)) {
        SkinnyArgs sa{M, N, K, (const uint8_t*)A, lda, (const uint8_t*)B, ldb, C, ldc};
        // one workgroup per 16-column block and 16-row slice of M; with
        // several slices the column blocks are padded to a multiple of 8
        const int64_t nblk = (N + kSkCols - 1) / kSkCols, slices = (M + 15) / 16;
        const int64_t blocks = slices == 1 ? nblk : (nblk + 7) / 8 * 8 * slices;
        if (blocks > 0x7FFFFFFF)
            return TG_ERR_NOT_SUPPORTED;
        const int split = skinny_split(blocks, K);
        if (split > 1 && c_dtype == TG_F32) {  // narrow N: split K over workgroups too
            hipLaunchKernelGGL(zero_f32<>, dim3((uint32_t)((N + 1023) / 1024), (uint32_t)M), dim3(256), 0, s, (float*)C, N, ldc);
            launch_skinny<E, O_F32, true>(sa, blocks, split, s);
            return launched();
        }
        switch (c_dtype) {
        case TG_F32: launch_skinny<E, O_F32>(sa, blocks, 1, s); break;
        case TG_F16: launch_skinny<E, O_F16>(sa, blocks, 1, s); break;
        default: launch_skinny<E, O_BF16>(sa, blocks, 1, s); break;
        }
        return launched();
    }
    TileArgs a{};
    a.M = M;
    a.N = N;
    a.K = K;
    a.A = (const uint8_t*)A;
    a.lda = lda;
    a.B = (const uint8_t*)B;
    a.ldb = ldb;
    a.C = C;
    a.ldc = ldc;
    a.alpha = 1.0f;
    if (b_layout == TG_COL_MAJOR)
        return launch_dense<E, B_KCONTIG>(a, c_dtype, s);
    return launch_dense<E, B_NCONTIG>(a, c_dtype, s);
}

}  // namespace tg
