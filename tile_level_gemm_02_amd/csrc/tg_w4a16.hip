// tg_gemm_w4a16 and tg_dequant_w4 (contract in include/tg.h).  Both run the
// same device routine, tg::dequant_w4_word, so the GEMM's weights are
// bit-identical to what tg_dequant_w4 writes.
#include "tg_gemm_w4.hpp"
#include "tg_gemm_w4s.hpp"
#include "tg_host.hpp"

namespace tg {

__global__ __launch_bounds__(256) void dequant_w4_kernel(DequantArgs p)
{
    const int64_t words = p.K / 8;
    const int64_t total = p.N * words;
    const W4Consts wc = w4_consts(p.zero_point);
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        const int64_t n = t / words, w = t - n * words;
        const uint32_t q = p.qw[n * p.ldq + w];
        const _Float16 s = bit_cast<_Float16>(p.scales[n * p.lds + (w * 8) / p.group_size]);
        *(u32x4*)(p.W + n * p.ldw + w * 8) = dequant_w4_word(q, wc, f16x2{s, s});
    }
}

}  // namespace tg

namespace {

tg_status check_w4(int64_t N, int64_t K, const int32_t* qweight, int64_t ldq, const void* scales,
                   int64_t lds, int32_t group_size, int32_t zero_point)
{
    if (N < 0 || K < 0)
        return TG_ERR_INVALID_VALUE;
    if (!tg::dims_fit(N, K, ldq, lds))
        return TG_ERR_NOT_SUPPORTED;
    if (group_size != 128 || (K % 128) != 0 || zero_point < 0 || zero_point > 15)
        return TG_ERR_NOT_SUPPORTED;
    if (N > 0 && K > 0) {
        if (qweight == nullptr || scales == nullptr)
            return TG_ERR_INVALID_VALUE;
        if (ldq < K / 8 || lds < K / group_size)
            return TG_ERR_INVALID_VALUE;
        if (!tg::aligned16(qweight) || ((ldq * 4) & 15) || ((uintptr_t)scales & 1u))
            return TG_ERR_MISALIGNED;
    }
    return TG_OK;
}

// gemm_w4 takes K in whole pairs of scale groups, up to its LDS capacity for
// scales (it fetches a column's scales as aligned 4-byte pairs), and
// addresses each operand through a buffer resource of kNumRecords bytes based
// at its tile's first row: every offset it forms, including the out-of-range
// marker added to one, must stay below 2^32.
bool w4_direct_eligible(const tg::TileArgs& a)
{
    if (a.K % 256 != 0 || a.K > 128 * tg::kW4MaxGroups || ((uintptr_t)a.scales & 3u) != 0 ||
        (a.lds & 1) != 0)
        return false;
    const int64_t lim = (int64_t)tg::kNumRecords;
    const int64_t kpast = a.K + 16 * 128;  // with the steps issued past the last one
    return 64 * a.lda * 2 + kpast * 2 < lim && 128 * a.ldq * 4 + kpast / 2 < lim &&
           128 * a.lds * 2 + a.K / 64 < lim;
}

// skinny_w4 addresses each operand through a buffer resource of kNumRecords
// bytes (A from its first row, qweight and scales from the workgroup's first
// column): every valid offset, per-lane part plus group part, must stay below
// that bound.
bool w4_skinny_eligible(const tg::TileArgs& a, int cols)
{
    const int64_t lim = (int64_t)tg::kNumRecords;
    return a.M * a.lda * 2 + a.K * 2 < lim && cols * a.ldq * 4 + a.K / 2 < lim && cols * a.lds * 2 + a.K / 64 < lim;
}

// Launch shape of skinny_w4_lds for AI A-copy instructions per stage: four
// waves with a two-slot ring each (a stage in flight while the previous one
// is multiplied), 16 columns per workgroup when A is at most 4 rows and 32
// above, where the A copies, shared by the workgroup's columns, cost more
// than the extra workgroups gain (measured at N = K = 8192).
// Batches up to this many rows take the decode kernel, in slices of 16 rows
// (each slice re-reads the weights, mostly from L2); above it the tile kernel.
// At N = K = 8192: 17-32 rows 27 us against 46 for the tile kernel, 48 rows
// 38 against 47, 64 rows 48.5 against 46.6.
constexpr int64_t kW4SliceMaxM = 48;

template <int AI> struct W4dCfg {
    static constexpr int WAVES = 4, RING = 2, NT = AI <= 2 ? 1 : 2;
};

// skinny_w4_lds: whole stages of two scale groups per wave (K a multiple of
// 2 * 128 * waves), scales copied as aligned 4-byte pairs, and the same
// buffer-offset bound as skinny_w4 for its 16 A rows and `cols` columns,
// with the stage offsets the ring forms past the end of K.
bool w4_skinny_lds_eligible(const tg::TileArgs& a, int waves, int cols, int ring)
{
    if (a.K <= 0 || a.K % (256 * waves) != 0 || ((uintptr_t)a.scales & 3u) != 0 || (a.lds & 1) != 0)
        return false;
    const int64_t lim = (int64_t)tg::kNumRecords;
    const int64_t past = 2 * (int64_t)ring;  // groups past the end of K
    return 16 * a.lda * 2 + (a.K + past * 128) * 2 < lim && cols * a.ldq * 4 + (a.K + past * 128) / 2 < lim &&
           cols * a.lds * 2 + (a.K / 128 + past) * 2 < lim;
}

// launches the LDS decode kernel for AI A-copy instructions per stage, or
// returns false (nothing launched) if the problem does not fit its shape.
// One row with each wave's K range at most kW4PreMaxKW takes the variant
// that copies A and the scales once per wave (PRE).
template <int AI>
bool launch_skinny_lds(const tg::TileArgs& a, hipStream_t s, tg_status* st)
{
    typedef W4dCfg<AI> G;
    constexpr int COLS = tg::W4dLayout<AI, G::NT>::COLS;
    if (!w4_skinny_lds_eligible(a, G::WAVES, COLS, G::RING))
        return false;

    // one workgroup per column block and 16-row slice of M; with several
    // slices the column blocks are padded to a multiple of 8 (see the kernel)
    const int64_t nblk = (a.N + COLS - 1) / COLS, slices = (a.M + 15) / 16;
    const int64_t blocks = slices == 1 ? nblk : (nblk + 7) / 8 * 8 * slices;
    if (blocks > 0x7FFFFFFF) {
        *st = TG_ERR_NOT_SUPPORTED;
        return true;
    }
    if constexpr (AI == 1 && G::NT == 1) {
        if (a.M == 1 && a.K / G::WAVES <= tg::kW4PreMaxKW) {
            hipLaunchKernelGGL((tg::skinny_w4_lds<AI, G::WAVES, G::RING, G::NT, true>), dim3((uint32_t)blocks),
                               dim3(G::WAVES * 64), 0, s, a);
            *st = tg::launched();
            return true;
        }
    }
    hipLaunchKernelGGL((tg::skinny_w4_lds<AI, G::WAVES, G::RING, G::NT>), dim3((uint32_t)blocks), dim3(G::WAVES * 64), 0,
                       s, a);
    *st = tg::launched();
    return true;
}

// The split kernel gemm_w4s (128 x 128 tiles, K split over S workgroups per
// tile through a workspace): S = the workgroups that fill the chip in one
// round (256 / tiles), at most 8, with every split holding whole pairs of
// scale groups, at least 8 and at most kW4sMaxGroups of them.  Used above
// the decode batch sizes, for K a multiple of 256 with 4-byte aligned
// scales of even stride, and 32-bit buffer offsets over a tile; 1 = no split.
int w4s_splits(int64_t M, int64_t N, int64_t K)
{
    if (M <= kW4SliceMaxM || N <= 0 || K <= 0 || K % 256 != 0 || !tg::dims_fit(M, N, K))
        return 1;
    const int64_t tiles = tg::n_tiles<128, 128>(M, N), G = K / 128;
    if (tiles >= 256 || tiles > tg::kSplitMaxCounters)
        return 1;
    int64_t S = 256 / tiles;
    if (S > 8)
        S = 8;
    while (S > 1 && G / S < 8)
        --S;
    if (S > 1 && (G + S - 1) / S + 2 > tg::kW4sMaxGroups)
        return 1;
    return (int)S;
}

int64_t w4s_ws_bytes(int64_t M, int64_t N, int64_t K)
{
    const int S = w4s_splits(M, N, K);
    return S <= 1 ? 0 : tg::kSplitCounterBytes + tg::n_tiles<128, 128>(M, N) * S * 128 * 128 * 4;
}

bool w4s_offsets_fit(const tg::TileArgs& a)
{
    if (((uintptr_t)a.scales & 3u) != 0 || (a.lds & 1) != 0)
        return false;
    const int64_t lim = (int64_t)tg::kNumRecords;
    return 128 * a.lda * 2 + a.K * 2 + 2048 < lim && 128 * a.ldq * 4 + a.K / 2 + 512 < lim &&
           128 * a.lds * 2 + a.K / 64 < lim;
}

tg_status w4a16_impl(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const int32_t* qweight, int64_t ldq,
                     const void* scales, int64_t lds, int32_t group_size, int32_t zero_point, void* C, int64_t ldc,
                     void* ws, int64_t ws_bytes, void* stream);

}  // namespace

extern "C" int64_t tg_gemm_w4a16_ex_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    return w4s_ws_bytes(M, N, K);
}

extern "C" tg_status tg_gemm_w4a16_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                      const int32_t* qweight, int64_t ldq, const void* scales, int64_t lds,
                                      int32_t group_size, int32_t zero_point, void* C, int64_t ldc, void* workspace,
                                      int64_t workspace_bytes, void* stream)
{
    if (workspace_bytes < 0 || (workspace == nullptr && workspace_bytes != 0))
        return TG_ERR_INVALID_VALUE;
    if (workspace != nullptr) {
        if (((uintptr_t)workspace & 255u) != 0)
            return TG_ERR_MISALIGNED;
        const int64_t need = tg_gemm_w4a16_ex_workspace_bytes(M, N, K);
        if (need < 0 || workspace_bytes < need)
            return TG_ERR_INVALID_VALUE;
    }
    return w4a16_impl(M, N, K, A, lda, qweight, ldq, scales, lds, group_size, zero_point, C, ldc, workspace,
                      workspace_bytes, stream);
}

extern "C" tg_status tg_gemm_w4a16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                   const int32_t* qweight, int64_t ldq, const void* scales,
                                   int64_t lds, int32_t group_size, int32_t zero_point, void* C,
                                   int64_t ldc, void* stream)
{
    return w4a16_impl(M, N, K, A, lda, qweight, ldq, scales, lds, group_size, zero_point, C, ldc, nullptr, 0, stream);
}

namespace {

tg_status w4a16_impl(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const int32_t* qweight, int64_t ldq,
                     const void* scales, int64_t lds, int32_t group_size, int32_t zero_point, void* C, int64_t ldc,
                     void* ws, int64_t ws_bytes, void* stream)
{
    if (M < 0)
        return TG_ERR_INVALID_VALUE;
    if (!tg::dims_fit(M, lda, ldc))
        return TG_ERR_NOT_SUPPORTED;
    tg_status st = check_w4(N, K, qweight, ldq, scales, lds, group_size, zero_point);
    if (st != TG_OK)
        return st;
    if (M == 0 || N == 0)
        return TG_OK;
    if (C == nullptr || ldc < N)
        return TG_ERR_INVALID_VALUE;
    if (K > 0) {
        if (A == nullptr || lda < K)
            return TG_ERR_INVALID_VALUE;
        if (!tg::aligned16(A) || ((lda * 2) & 15))
            return TG_ERR_MISALIGNED;
    }
    if (!tg::aligned16(C) || ((ldc * 2) & 15))
        return TG_ERR_MISALIGNED;
    tg::TileArgs a{};
    a.M = M;
    a.N = N;
    a.K = K;
    a.A = (const uint8_t*)A;
    a.lda = lda;
    a.C = C;
    a.ldc = ldc;
    a.alpha = 1.0f;
    a.group_m = 4;
    a.qw = (const uint32_t*)qweight;
    a.ldq = ldq;
    a.scales = (const uint16_t*)scales;
    a.lds = lds;
    a.zero_point = zero_point;
    hipStream_t s = (hipStream_t)stream;
    if (ws != nullptr) {  // the split kernel, where its plan pays and its workspace fits
        const int S = w4s_splits(M, N, K);
        if (S > 1 && w4s_ws_bytes(M, N, K) <= ws_bytes && w4s_offsets_fit(a)) {
            const int64_t tiles = tg::n_tiles<128, 128>(M, N);
            a.splits = (uint32_t)S;
            a.counters = (uint32_t*)ws;
            a.partials = (float*)((uint8_t*)ws + tg::kSplitCounterBytes);
            hipLaunchKernelGGL((tg::gemm_w4s<6>), dim3((uint32_t)(tiles * S)), dim3(tg::kW4sThreads), 0, s, a);
            return tg::launched();
        }
    }
    if (M <= kW4SliceMaxM) {  // decode: a weight stream, too few output tiles to fill the chip
        tg_status lst = TG_OK;
        if ((M <= 2 && launch_skinny_lds<1>(a, s, &lst)) || (M > 2 && M <= 4 && launch_skinny_lds<2>(a, s, &lst)) ||
            (M > 4 && M <= 8 && launch_skinny_lds<4>(a, s, &lst)) || (M > 8 && launch_skinny_lds<8>(a, s, &lst)))
            return lst;
    }
    constexpr int WAVES = 8, NT = 2, UNR = 1;  // decode kernel: 16*NT columns per workgroup
    if (M <= 16 && w4_skinny_eligible(a, 16 * NT)) {  // decode: a weight stream, too few output tiles
        const int64_t blocks = (N + 16 * NT - 1) / (16 * NT);
        if (blocks > 0x7FFFFFFF)
            return TG_ERR_NOT_SUPPORTED;
        hipLaunchKernelGGL((tg::skinny_w4<WAVES, NT, UNR>), dim3((uint32_t)blocks), dim3(WAVES * 64), 0, s, a);
        return tg::launched();
    }
    if (w4_direct_eligible(a)) {
        constexpr int BM = 64, BN = 128, NA = 4;
        const int64_t tiles = tg::n_tiles<BM, BN>(M, N);
        if (tiles > 0x7FFFFFFF)
            return TG_ERR_NOT_SUPPORTED;
        hipLaunchKernelGGL((tg::gemm_w4<BM, NA>), dim3((uint32_t)tiles), dim3(tg::kW4Threads), 0, s, a);
        return tg::launched();
    }
    if (tg::n_tiles<128, 128>(M, N) >= 96)
        return tg::launch_tile<tg::E_F16, tg::B_KCONTIG, tg::O_F16, 128, 128, true>(a, s);
    return tg::launch_tile<tg::E_F16, tg::B_KCONTIG, tg::O_F16, 64, 64, true>(a, s);
}

}  // namespace

extern "C" tg_status tg_dequant_w4(int64_t N, int64_t K, const int32_t* qweight, int64_t ldq,
                                   const void* scales, int64_t lds, int32_t group_size,
                                   int32_t zero_point, void* W, int64_t ldw, void* stream)
{
    tg_status st = check_w4(N, K, qweight, ldq, scales, lds, group_size, zero_point);
    if (st != TG_OK)
        return st;
    if (N == 0 || K == 0)
        return TG_OK;
    if (!tg::dims_fit(ldw, 0, 0))
        return TG_ERR_NOT_SUPPORTED;
    if (W == nullptr || ldw < K)
        return TG_ERR_INVALID_VALUE;
    if (!tg::aligned16(W) || ((ldw * 2) & 15))
        return TG_ERR_MISALIGNED;
    tg::DequantArgs d{N, K, (const uint32_t*)qweight, ldq, (const uint16_t*)scales, lds,
                      group_size, zero_point, (uint16_t*)W, ldw};
    const int64_t words = N * (K / 8);
    int64_t blocks = (words + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;  // grid-stride loop covers the rest
    hipLaunchKernelGGL(tg::dequant_w4_kernel, dim3((uint32_t)blocks), dim3(256), 0,
                       (hipStream_t)stream, d);
    return tg::launched();
}
