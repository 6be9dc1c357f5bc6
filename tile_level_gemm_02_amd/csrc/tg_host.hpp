// Host-side helpers of the C ABI: argument validation and kernel launch.
// Validation runs before any HIP call, so a rejected call launches nothing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_abi.hpp"
#include "tg_gemm_nt.hpp"
#include "tg_gemm_skinny.hpp"
#include "tg_kernels.hpp"

namespace tg {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0u; }

inline int out_bytes(int d) { return d == TG_F32 ? 4 : 2; }

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
    if (!dims_fit(M, N, K, lda, ldb, ldc))
        return TG_ERR_NOT_SUPPORTED;
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
    if (!aligned16(C) || ((ldc * out_bytes(c_dtype)) & 15))
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

// Tile edge for the NT kernel: pick_tile's, except that where the 128 tile
// would take more than one round of the chip (over 256 tiles, which leaves
// it the 4-slot ring that waits on copies) the 256 tile runs instead, unless
// it pads the output by more than a quarter over the 128 tile's padding
// (fp8: only from 128 tiles of 256 on).  Back to back, old -> new: bf16
// 2304^3 54.7 -> 48.5 us, 3072^3 101.7 -> 66.4, 3328^3 116.8 -> 78.8,
// 3072 x 3072 x 1024 40.9 -> 27.0, 1024 x 8192 x 4096 87.2 -> 77.7 (B
// row-major alike); fp8 3072^3 59.2 -> 41.4, 3328^3 69.4 -> 49.1, while at
// 81 tiles of 256 (2176^3, 2304^3) its 128 tile stayed faster.
template <int EB>
inline int pick_tile_nt(int64_t M, int64_t N)
{
    const int t = pick_tile(M, N, true);
    const int64_t t128 = n_tiles<128, 128>(M, N), t256 = n_tiles<256, 256>(M, N);
    if (t == 128 && t128 > 256 && t256 * 4 * 4 <= t128 * 5 && (EB == 2 || t256 >= 128))
        return 256;
    return t;
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
// the ring of the 256 x 256 tile.  fp8 takes five (2.5 K steps in flight:
// its copies miss L2 more often and wait longer; ~9% faster at 8192^3).  For
// 16-bit inputs five (all 160 KiB of LDS) against four: with the operands
// outside the Infinity Cache (flushed launches) five ran 2-14% faster —
// 3072^3 76.5 -> 65.9 us, 3584^3 91.3 -> 82.3, 4096^3 111.2 -> 108.5 — but
// back to back (operands cached) 1-2% slower: 4096^3 102.4 -> 104.2, 8192^3
// 773 -> 783.  A launch of fewer than 256 tiles runs in one round, all of it
// on cold operands when they come from HBM, so it takes five; a full round
// or more (4096^3 and up, where later rounds find the operands cached)
// keeps four.
template <int E> struct NtStaging { static constexpr int RB = 128; };
template <int E, int BM> struct NtRing { static constexpr int NH = 4; };
template <> struct NtRing<E_FP8, 256> { static constexpr int NH = 5; };
template <int E>
inline int nt_ring256(int64_t tiles)
{
    return E == E_FP8 || tiles < 256 ? 5 : NtRing<E, 256>::NH;
}

// Waves of the NT kernel per tile: the 256 x 256 tile takes 8 (2 x 4, two
// per SIMD) for the LDS read rate its fragments need; smaller tiles take 4.
// For fp8 the 256 tile takes 4 (128 x 128 per wave, one per SIMD: a third
// less LDS reading per step, its 256 accumulators in AGPRs, 16 registers
// spilled): measured with the two builds interleaved, 8192^3 460 -> 422 us,
// 16384 x 8192 x 8192 834 -> 789, 4096 x 4096 x 16384 197 -> 189, and
// 0.3-3% faster at the other shapes tried, bit-identical.  (For 16-bit
// inputs the two layouts measured the same.)
template <int E, int BM, int BN> struct NtWaves { static constexpr int WM = 2, WN = 2; };
template <int E> struct NtWaves<E, 256, 256> { static constexpr int WM = 2, WN = 4; };
template <> struct NtWaves<E_FP8, 256, 256> { static constexpr int WM = 2, WN = 2; };

inline int nt_waves(int tile) { return tile == 256 ? 8 : 4; }  // (the most for this edge: counters per tile)

// ---- K split over workgroups (only with a caller workspace)
//
// Workspace of a split launch: the first kSplitCounterBytes hold 32-bit
// arrival counters, one per tile and wave of the launch (zero before the
// first call, left zero by every call), so one zero fill of a workspace
// serves every later call whatever its shape; then one fp32 partial share
// per tile, split and wave (tile x tile floats per tile and split), scratch
// that needs no clearing.
constexpr int64_t kSplitCounterBytes = 65536;
constexpr int64_t kSplitMaxCounters = kSplitCounterBytes / 4;

inline int64_t split_ws_bytes(int64_t tiles, int splits, int64_t tile_elems)
{
    return splits <= 1 ? 0 : kSplitCounterBytes + tiles * splits * tile_elems * 4;
}

// The tiles of a short last round, run without a split in a second launch:
// each 256 x 256 tile as 2 parts of 256 x 128, 4 of 128 x 128 or 16 of
// 64 x 64, the smallest parts whose launch fits one round of 256 workgroups.
enum NtTail : int { kTailNone = 0, kTailWide = 1, kTail128 = 2, kTail64 = 3 };

// Launch plan of the NT kernel: tile edge, LDS ring depth, K split.
struct NtPlan {
    int tile, nh, splits;
    int64_t ws_bytes;  // workspace the plan needs (0 without a split)
    int64_t dp;        // > 0: this many tiles run whole, the rest split `splits` ways
    int tn;            // the tile's N edge: `tile`, or 128 for the 256 x 128 tile
    int tail;          // 256 tile: the first dp tiles whole, then the rest in parts (NtTail)
};

// Estimated cycles of one compute unit for an NT launch with tile edge T and
// S workgroups per tile.  A workgroup's K loop is bound by the larger of its
// L2 -> LDS copies (about 37 bytes per clock per CU, measured) and its MFMA
// issue (4096 FLOP per clock per CU, 8192 for fp8); a split adds the store
// of each partial share and, for the last arrival, the loads of the other
// S - 1 and its own (device-coherent accesses, about 16 bytes per clock per
// CU as fitted to splits measured at N = K = 8192); workgroups run in rounds
// of one per CU.
inline double nt_round_cost(int64_t K, int EB, int T, int S)
{
    const double kw = (double)K / S;  // K elements per workgroup
    const double copy = 2.0 * T * kw * EB / 37.0;
    const double mfma = 2.0 * T * T * kw / (EB == 1 ? 8192.0 : 4096.0);
    const double red = S > 1 ? (double)T * T * 4.0 * (S + 1) / 16.0 : 0.0;
    const double fixed = 4000.0;  // ring fill and epilogue
    return (copy > mfma ? copy : mfma) + red + fixed;
}

// Cycles of one compute unit for a 256 x 256 tile running K / S of K in the
// last round of a launch that splits only that round (S = 1: a whole tile):
// the K loop at the rate measured for this tile, about 1.17 times its MFMA
// issue time; the ring fill and epilogue; with S > 1 about 16 K cycles per
// split for the hand-off of the 256 KiB partial tiles (fitted to last-round
// splits timed back to back at 4608^3, 6144^3, 7168^3, 9216 x 9216 x 4096,
// 4300 x 4104 x 8200 and 3000 x 6000 x 4096: the split count this picks ran
// fastest, or within 1% of it, at each).
inline double nt_round256_cost(int64_t K, int EB, int S)
{
    const double kw = (double)K / S;
    const double copy = 2.0 * 256 * kw * EB / 37.0;
    const double mfma = 2.0 * 256 * 256 * kw / (EB == 1 ? 8192.0 : 4096.0);
    return 1.17 * (copy > mfma ? copy : mfma) + 4000.0 + (S > 1 ? 16384.0 * S : 0.0);
}

inline double nt_cost(int64_t M, int64_t N, int64_t K, int EB, int T, int S)
{
    const double tiles = (double)(((M + T - 1) / T) * ((N + T - 1) / T));
    const double rounds = (double)((int64_t)(tiles * S + 255.0) / 256);
    return rounds * nt_round_cost(K, EB, T, S);
}

// The 256 x 128 tile (4 waves of 128 x 64): where it makes one round of
// more than 128 workgroups, the tiles of 256 x 256 leave compute units idle
// and those of 128 x 128 need more than a round; unless it pads the output a
// quarter more than the 128 tile.  Back to back, against the square tiles'
// best: bf16 2304^3 48.5 -> 37.1 us, 2560^3 54.6 -> 41.4, 2816^3 60.4 ->
// 46.7, 2816 x 2816 x 1024 27.2 -> 21.0, 1024 x 8192 x 4096 76.7 -> 61.9
// (B row-major alike: 2560^3 52.9 -> 39.8); fp8 2304^3 30.1 -> 21.0,
// 2304 x 2304 x 8192 89.1 -> 54.5, 1536 x 3072 x 4096 47.4 -> 30.6 (B
// row-major alike).  At 128 of its tiles (2048^3) the 128 tile's one round
// stays faster (bf16 21.4 against 31.8 us), and past 256 the 256 tile
// (3072^3: 64.4 against 90.4).
// Ring depth of the 256 x 128 tile: six half-stages (three K steps in
// flight; its A and B slots of 32 and 16 KiB take 144 KiB).
constexpr int kWideNH = 6;

template <int EB, int BL>
inline bool nt_wide(int64_t M, int64_t N)
{
    const int64_t tw = n_tiles<256, 128>(M, N), t128 = n_tiles<128, 128>(M, N);
    return tw > 128 && tw <= 256 && tw * 8 <= t128 * 5;
}

template <int E, int BL>
NtPlan plan_nt(int64_t M, int64_t N, int64_t K, bool allow_split)
{
    constexpr int EB = ElemInfo<E>::bytes;
    if (nt_wide<EB, BL>(M, N))  // (one round of its tiles: a K split would not fit the chip)
        return NtPlan{256, kWideNH, 1, 0, 0, 128, 0};
    NtPlan p{pick_tile_nt<EB>(M, N), 4, 1, 0, 0, 0, 0};
    if (EB == 1 && BL == B_NCONTIG && p.tile < 128)
        p.tile = 128;  // (nt_eligible_nrow only admits shapes that pick 128 or 256)
    if (allow_split) {
        // split candidates on every tile edge, each workgroup keeping at least
        // 8 K steps, against the unsplit default
        const int64_t KT = (K + 128 / EB - 1) / (128 / EB);
        double best = nt_cost(M, N, K, EB, p.tile, 1);
        // (the 256 tile's 256 KiB partial shares cost more to reduce than its
        // splits save: measured slower at every M from 320 to 3072, N = K = 8192)
        for (int T = 64; T <= 128; T *= 2) {
            if (EB == 1 && BL == B_NCONTIG && T < 128)
                continue;
            if (((M + T - 1) / T) * ((N + T - 1) / T) * nt_waves(T) > kSplitMaxCounters)
                continue;
            // (only splits that fit the chip in one round: at N = K = 8192,
            // M = 768, 768 split workgroups measured 8% slower than 384 unsplit)
            const int64_t tiles_t = ((M + T - 1) / T) * ((N + T - 1) / T);
            for (int S = 2; S <= 8 && KT / S >= 8 && tiles_t * S <= 256; ++S) {
                const double c = nt_cost(M, N, K, EB, T, S);
                if (c < best * 0.97) {  // (a clear gain over the unsplit default)
                    best = c;
                    p.tile = T;
                    p.splits = S;
                }
            }
        }
        // More than one round of 256 tiles with a short last round: the full
        // rounds run whole tiles and the last round's R tiles split K S ways
        // (R * S <= 256 workgroups, dispatched right behind the whole tiles).
        // Taken for 16-bit inputs with 65 to 128 tiles left over; fewer, and
        // fp8, run faster as the parts of a second launch (NtTail, below):
        // bf16 4608^3 (68 left) split 183.3 against parts 189.6 us, but
        // 6144^3 (64 left) 396.6 against 376.9 and fp8 6144^3 249.6 against
        // 190.2 (flushed).
        if (p.tile == 256 && p.splits == 1 && EB == 2) {
            const int64_t tiles256 = ((M + 255) / 256) * ((N + 255) / 256);
            const int64_t D = tiles256 / 256 * 256, R = tiles256 - D;
            if (D > 0 && R > 64 && R * 2 <= 256 && R * nt_waves(256) <= kSplitMaxCounters) {
                const double whole = (double)(D / 256) * nt_round256_cost(K, EB, 1);
                const double unsplit = whole + nt_round256_cost(K, EB, 1);
                double hbest = unsplit;
                int hs = 1;
                for (int S = 2; R * S <= 256 && KT / S >= 8; ++S) {
                    const double c = whole + nt_round256_cost(K, EB, S);
                    if (c < hbest) {
                        hbest = c;
                        hs = S;
                    }
                }
                if (hs > 1 && hbest < unsplit * 0.97) {  // (a clear gain over the whole-tile last round)
                    p.splits = hs;
                    p.dp = D;
                }
            }
        }
    }
    // A short last round without a split: its tiles run in parts (NtTail)
    // in a second launch, which shortens the round; no workspace is needed.
    if (p.tile == 256 && p.splits == 1) {
        const int64_t tiles256 = ((M + 255) / 256) * ((N + 255) / 256);
        const int64_t D = tiles256 / 256 * 256, R = tiles256 - D;
        if (D > 0 && R > 0 && R * 2 <= 256) {
            p.dp = D;
            const bool no64 = EB == 1 && BL == B_NCONTIG;  // (64-byte fp8 B rows: no 64 tile)
            p.tail = R * 16 <= 256 && !no64 ? kTail64 : R * 4 <= 256 ? kTail128 : kTailWide;
        }
    }
    const int64_t tiles = p.dp > 0 ? ((M + 255) / 256) * ((N + 255) / 256) - p.dp
                                   : ((M + p.tile - 1) / p.tile) * ((N + p.tile - 1) / p.tile);
    // ring depth: the 256 tile per element type; the 128 and 64 tiles take 8
    // half-stages (4 steps in flight) when their workgroups fit the chip at
    // the occupancy that allows (one 128 KiB workgroup, or two of 64 KiB, per
    // CU), else 4, which leaves room for more resident workgroups.  A small
    // tile does little MFMA work per K step, so with 2 steps in flight it
    // waits on copy latency: at N = K = 8192, M = 128 (64 tiles) 96 -> 45 us,
    // M = 256 (128 tiles) 114 -> 77 us; 2048^3 27 -> 21 us.
    if (p.tile == 256)
        p.nh = p.dp > 0 ? nt_ring256<E>(tiles + p.dp) : nt_ring256<E>(tiles);
    else if (p.tile == 64)
        p.nh = 8;
    else
        p.nh = tiles * p.splits <= 256 ? 8 : 4;
    p.tn = p.tile;
    p.ws_bytes = split_ws_bytes(tiles, p.splits, (int64_t)p.tile * p.tile);  // (split tiles only)
    return p;
}

template <int E, int O, int BM, int BN, int BL, int NH>
tg_status launch_nt(const TileArgs& a, int splits, hipStream_t s, int64_t grid_override = 0)
{
    const int64_t tiles = n_tiles<BM, BN>(a.M, a.N);
    const int64_t grid = grid_override > 0 ? grid_override : a.dp > 0 ? a.dp + (tiles - a.dp) * splits : tiles * splits;
    if (grid > 0x7FFFFFFF)
        return TG_ERR_NOT_SUPPORTED;
    constexpr int RB = NtStaging<E>::RB;
    constexpr int WM = NtWaves<E, BM, BN>::WM, WN = NtWaves<E, BM, BN>::WN;
    hipLaunchKernelGGL((gemm_nt<E, O, BM, BN, RB, NH, WM, WN, BL>), dim3((uint32_t)grid), dim3(64 * WM * WN), 0, s, a);
    return launched();
}

// Launch an NT plan.  With plan.splits > 1, `ws` is a zeroed-counter
// workspace of at least plan.ws_bytes bytes (256-byte aligned).
template <int E, int O, int BL>
tg_status launch_nt_plan(TileArgs& a, const NtPlan& plan, void* ws, hipStream_t s)
{
    a.group_m = 4;
    a.splits = (uint32_t)plan.splits;
    a.dp = (uint32_t)plan.dp;
    if (plan.splits > 1) {
        a.counters = (uint32_t*)ws;
        a.partials = (float*)((uint8_t*)ws + kSplitCounterBytes);
    }
    if (plan.tail != kTailNone) {
        // the first plan.dp tiles of 256 x 256 whole, then every later tile of
        // the walk in parts, in a second launch
        const int64_t rest = n_tiles<256, 256>(a.M, a.N) - plan.dp;
        TileArgs b = a;
        a.dp = (uint32_t)plan.dp;
        tg_status st = plan.nh == 5 ? launch_nt<E, O, 256, 256, BL, 5>(a, 1, s, plan.dp)
                                    : launch_nt<E, O, 256, 256, BL, 4>(a, 1, s, plan.dp);
        if (st != TG_OK)
            return st;
        b.dp = 0;
        b.splits = 1;
        b.sub256 = (uint32_t)plan.dp + 1u;
        if (plan.tail == kTailWide)
            return launch_nt<E, O, 256, 128, BL, kWideNH>(b, 1, s, 2 * rest);
        if (plan.tail == kTail128)
            return launch_nt<E, O, 128, 128, BL, 8>(b, 1, s, 4 * rest);
        if constexpr (ElemInfo<E>::bytes == 1 && BL == B_NCONTIG)
            return TG_ERR_NOT_SUPPORTED;  // (never planned)
        else
            return launch_nt<E, O, 64, 64, BL, 8>(b, 1, s, 16 * rest);
    }
    if (plan.tile == 256 && plan.tn == 128) {
        if (plan.nh == 6)
            return launch_nt<E, O, 256, 128, BL, 6>(a, plan.splits, s);
        return launch_nt<E, O, 256, 128, BL, 4>(a, plan.splits, s);
    }
    if (plan.tile == 256) {
        if (plan.nh == 5)
            return launch_nt<E, O, 256, 256, BL, 5>(a, plan.splits, s);
        return launch_nt<E, O, 256, 256, BL, 4>(a, plan.splits, s);
    }
    if (plan.tile == 128) {
        if (plan.nh == 8)
            return launch_nt<E, O, 128, 128, BL, 8>(a, plan.splits, s);
        return launch_nt<E, O, 128, 128, BL, 4>(a, plan.splits, s);
    }
    if constexpr (ElemInfo<E>::bytes == 1 && BL == B_NCONTIG)
        return TG_ERR_NOT_SUPPORTED;  // (never planned: 64-byte fp8 B rows)
    else
        return launch_nt<E, O, 64, 64, BL, 8>(a, plan.splits, s);
}

// Whether the NT kernel takes this problem, for either layout of B.
template <int E, int BL>
inline bool nt_takes(const TileArgs& a)
{
    if constexpr (BL == B_KCONTIG)
        return nt_eligible<E>(a);
    else
        return nt_eligible_nrow<E>(a);
}

// Dense GEMM launch.  `ws`/`ws_bytes`: a caller workspace (NULL/0 for none);
// the NT kernel splits K over workgroups only when the plan's workspace fits.
template <int E, int BL>
tg_status launch_dense(TileArgs& a, int c_dtype, hipStream_t s, void* ws = nullptr, int64_t ws_bytes = 0)
{
    if (nt_takes<E, BL>(a)) {
        NtPlan plan = plan_nt<E, BL>(a.M, a.N, a.K, ws != nullptr);
        if (plan.ws_bytes > ws_bytes)
            plan = plan_nt<E, BL>(a.M, a.N, a.K, false);
        switch (c_dtype) {
        case TG_F32: return launch_nt_plan<E, O_F32, BL>(a, plan, ws, s);
        case TG_F16: return launch_nt_plan<E, O_F16, BL>(a, plan, ws, s);
        default: return launch_nt_plan<E, O_BF16, BL>(a, plan, ws, s);
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

// Workgroups per column block of the skinny kernel when N alone gives few:
// about one per CU (256 in all), each with at least 2048 of K.  Without a
// workspace (fp32 atomic adds into a C that a fill launch zeroes first) only
// a split into four or more pays for the fill.  Flushed launches, M = 16,
// K = 8192, 16-bit inputs: with a workspace N = 512 14.4 -> 10.7 us (4
// splits) and N = 2048 15.4 -> 13.5 us (2), where two workgroups per CU (8
// splits at N = 512, 4 at N = 2048) took 12.1 and 16.3 us; by atomics
// N = 1024 14.5 -> 13.0 us (4), while 2 or 3 splits ran 0.4-2.4 us slower
// than none at every N and K measured.
inline int skinny_split(int64_t blocks, int64_t K, bool atomic)
{
    int64_t split = 256 / blocks;
    const int64_t most = K / 2048;
    if (split > most)
        split = most;
    if (atomic && split < 4)
        split = 1;
    return split > 1 ? (int)split : 1;
}

// 16-column groups per skinny workgroup: two when M takes several 16-row
// slices (each slice's workgroups copy its A rows over all of K, so wider
// workgroups halve those bytes: bf16 N = K = 8192, flushed, M = 24 40.4 ->
// 36.5 us and M = 32 42.5 -> 38.3 us), one for a single slice (M = 16:
// 28.0 us against 28.3; two per CU of the narrower workgroups keep more
// copies in flight).
inline int skinny_cg(int64_t M) { return M > 16 ? 2 : 1; }

template <int E, int O, int AI, int SPLIT, int CG>
void launch_skinny_ai(const SkinnyArgs& sa, int64_t blocks, int split, hipStream_t s)
{
    typedef SkinnyCfg G;
    hipLaunchKernelGGL((skinny_gemm<E, O, G::WAVES, AI, G::RING, SPLIT, CG>), dim3((uint32_t)blocks, (uint32_t)split),
                       dim3(64 * G::WAVES), 0, s, sa);
}

// A rows are copied 8 at a time: one copy instruction for M <= 8, two above
// (16-row slices above 16).
template <int E, int O, int SPLIT = 0>
void launch_skinny(const SkinnyArgs& sa, int64_t blocks, int split, hipStream_t s)
{
    if (sa.M <= 8)
        launch_skinny_ai<E, O, 1, SPLIT, 1>(sa, blocks, split, s);
    else if (skinny_cg(sa.M) == 1)
        launch_skinny_ai<E, O, 2, SPLIT, 1>(sa, blocks, split, s);
    else
        launch_skinny_ai<E, O, 2, SPLIT, 2>(sa, blocks, split, s);
}

// Workspace of the skinny kernel's split through partial tiles: the
// counters (one per workgroup column and 16-column group), then a 1 KiB
// partial tile per workgroup and group; 0 where the counters would not fit
// their region.
inline int64_t skinny_ws_bytes(int64_t M, int64_t blocks, int split)
{
    const int64_t groups = skinny_cg(M);
    if (split <= 1 || blocks * groups > kSplitMaxCounters)
        return 0;
    return kSplitCounterBytes + blocks * groups * split * 1024;
}

// Workgroup columns of the skinny kernel: one per column block (16 *
// skinny_cg(M) columns) and 16-row slice of M; with several slices the
// column blocks are padded to a multiple of 8.
inline int64_t skinny_blocks(int64_t M, int64_t N)
{
    const int64_t cols = 16 * skinny_cg(M);
    const int64_t nblk = (N + cols - 1) / cols, slices = (M + 15) / 16;
    return slices == 1 ? nblk : (nblk + 7) / 8 * 8 * slices;
}

// Batches up to this many rows against a K-contiguous B take the skinny
// kernel, in 16-row slices (each slice re-reads B, mostly from L2).  At
// N = K = 8192 (bf16, flushed, 32 columns per workgroup): 17 rows 34 us,
// 32 rows 38, 33 rows 47 and 48 rows 50, against 53 for the tile kernel
// (without a workspace: no K split).  Where the NT kernel splits K over
// workgroups through a caller workspace it is faster from 33 rows on (36 us
// for 33-64 rows at N = K = 8192): there the skinny kernel stops at 32 rows.
constexpr int64_t kSkSliceMaxM = 48;
constexpr int64_t kSkSliceMaxMSplit = 32;

// Whether a dense 16-bit call with M rows takes the skinny kernel: up to
// kSkSliceMaxMSplit rows always, up to kSkSliceMaxM unless the NT kernel
// would split K with the workspace given.
template <int E>
bool skinny_takes(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int b_layout, const void* ws,
                  int64_t ws_bytes)
{
    if (M > kSkSliceMaxM || b_layout != TG_COL_MAJOR || K <= 0 ||
        !skinny_offsets_fit(K, lda, ldb, SkinnyCfg::RING, skinny_cg(M)))
        return false;
    if (M <= kSkSliceMaxMSplit || ws == nullptr)
        return true;
    TileArgs t{};
    t.M = M;
    t.N = N;
    t.K = K;
    t.lda = lda;
    t.ldb = ldb;
    if (!nt_eligible<E>(t))
        return true;
    const NtPlan plan = plan_nt<E, B_KCONTIG>(M, N, K, true);
    return !(plan.splits > 1 && plan.ws_bytes <= ws_bytes);
}

// fp16 / bf16 GEMM.  Few rows (kSkSliceMaxM) against a K-contiguous B take
// the skinny kernel; everything else the tile kernel (K == 0 runs it with no
// K steps, which stores zeros: the empty sum).
template <int E>
tg_status gemm_16bit(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, int b_layout, void* C, int64_t ldc, int c_dtype, void* stream,
                     void* ws = nullptr, int64_t ws_bytes = 0)
{
    bool empty;
    tg_status st = check_dense(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, 2, &empty);
    if (st != TG_OK || empty)
        return st;
    hipStream_t s = (hipStream_t)stream;
    typedef SkinnyCfg G;
    if (skinny_takes<E>(M, N, K, lda, ldb, b_layout, ws, ws_bytes)) {
        SkinnyArgs sa{M, N, K, (const uint8_t*)A, lda, (const uint8_t*)B, ldb, C, ldc};
        const int64_t blocks = skinny_blocks(M, N);
        if (blocks > 0x7FFFFFFF)
            return TG_ERR_NOT_SUPPORTED;
        // narrow N: split K over workgroups too
        const int split = skinny_split(blocks, K, false);
        const int64_t need = split > 1 ? skinny_ws_bytes(M, blocks, split) : 0;
        if (ws != nullptr && need > 0 && need <= ws_bytes) {
            // partial tiles in the workspace, the last arrival stores C: any output type
            sa.counters = (uint32_t*)ws;
            sa.partials = (float*)((uint8_t*)ws + kSplitCounterBytes);
            switch (c_dtype) {
            case TG_F32: launch_skinny<E, O_F32, 2>(sa, blocks, split, s); break;
            case TG_F16: launch_skinny<E, O_F16, 2>(sa, blocks, split, s); break;
            default: launch_skinny<E, O_BF16, 2>(sa, blocks, split, s); break;
            }
            return launched();
        }
        const int asplit = c_dtype == TG_F32 ? skinny_split(blocks, K, true) : 1;
        if (asplit > 1) {  // no workspace: fp32 atomic adds into a zeroed C
            hipLaunchKernelGGL(zero_f32<>, dim3((uint32_t)((N + 1023) / 1024), (uint32_t)M), dim3(256), 0, s, (float*)C,
                               N, ldc);
            launch_skinny<E, O_F32, 1>(sa, blocks, asplit, s);
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
        return launch_dense<E, B_KCONTIG>(a, c_dtype, s, ws, ws_bytes);
    return launch_dense<E, B_NCONTIG>(a, c_dtype, s, ws, ws_bytes);
}

// fp8 GEMM (validation as for the 16-bit inputs, plus finite scales).
inline tg_status gemm_fp8(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                          int64_t ldb, int b_layout, float scale_a, float scale_b, void* C, int64_t ldc,
                          int c_dtype, void* stream, void* ws = nullptr, int64_t ws_bytes = 0)
{
    bool empty;
    tg_status st = check_dense(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, 1, &empty);
    if (st != TG_OK || empty)
        return st;
    if (!__builtin_isfinite(scale_a) || !__builtin_isfinite(scale_b))
        return TG_ERR_INVALID_VALUE;
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
    a.alpha = scale_a * scale_b;
    hipStream_t s = (hipStream_t)stream;
    if (b_layout == TG_COL_MAJOR)
        return launch_dense<E_FP8, B_KCONTIG>(a, c_dtype, s, ws, ws_bytes);
    return launch_dense<E_FP8, B_NCONTIG>(a, c_dtype, s, ws, ws_bytes);
}

// Workspace a dense call would use for its K split: the skinny kernel's for
// few rows against a K-contiguous B, else the NT plan's for a problem on the
// NT kernel's element grid (whole 16-byte chunks along K, and along N for a
// row-major B); 0 where it never splits.
template <int E>
int64_t dense_ws_bytes(int64_t M, int64_t N, int64_t K, int b_layout)
{
    constexpr int CE = 16 / ElemInfo<E>::bytes;
    if (M <= 0 || N <= 0 || K <= 0 || !dims_fit(M, N, K))
        return 0;
    if (E != E_FP8 && M <= kSkSliceMaxMSplit && b_layout == TG_COL_MAJOR) {  // the skinny kernel (any K)
        const int64_t blocks = skinny_blocks(M, N);
        return skinny_ws_bytes(M, blocks, skinny_split(blocks, K, false));
    }
    if (K % CE != 0)
        return 0;
    if (b_layout == TG_COL_MAJOR)
        return plan_nt<E, B_KCONTIG>(M, N, K, true).ws_bytes;
    if (N % CE != 0)
        return 0;
    return plan_nt<E, B_NCONTIG>(M, N, K, true).ws_bytes;
}

// Per-type entry points with a split workspace, each defined (and its kernels
// instantiated) in that type's translation unit; tg_gemm_ex dispatches to them.
tg_status gemm_f16_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                      int b_layout, void* C, int64_t ldc, int c_dtype, void* stream, void* ws, int64_t ws_bytes);
tg_status gemm_bf16_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                       int b_layout, void* C, int64_t ldc, int c_dtype, void* stream, void* ws, int64_t ws_bytes);
tg_status gemm_fp8_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                      int b_layout, float scale_a, float scale_b, void* C, int64_t ldc, int c_dtype, void* stream,
                      void* ws, int64_t ws_bytes);
int64_t ws_bytes_f16(int64_t M, int64_t N, int64_t K, int b_layout);
int64_t ws_bytes_bf16(int64_t M, int64_t N, int64_t K, int b_layout);
int64_t ws_bytes_fp8(int64_t M, int64_t N, int64_t K, int b_layout);

}  // namespace tg
