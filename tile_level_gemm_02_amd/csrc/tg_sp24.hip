// tg_gemm_sp24_bf16: 2:4 structured-sparse GEMM (contract in include/tg.h).
#include "tg_gemm_sp.hpp"
#include "tg_host.hpp"

namespace {

// gemm_sp24 addresses each operand through a buffer resource of kNumRecords
// bytes based at its tile's first row: every offset it forms must stay below
// that bound.
bool sp24_offsets_fit(int64_t K, int64_t lda, int64_t ldv, int64_t ldm)
{
    const int64_t lim = (int64_t)tg::kNumRecords;
    return 256 * lda * 2 + K * 2 < lim && 256 * ldv * 2 + K < lim && 256 * ldm + K / 8 < lim;
}

// Waves per workgroup of gemm_sp24: 8.  Four (128 x 128 per wave, each
// wave issuing two copy slots' copies) gave bit-identical results but ran
// slower at every shape tried, interleaved on one lease: 4096^3 82.8 ->
// 108.9 us, 8192^3 571 -> 636, 2304^3 37.6 -> 48.5, 4100 x 4000 x 4160
// 146 -> 153.
constexpr int kSpWaves = 8;

template <bool CP4>
tg_status launch_sp24(const tg::SpArgs& a, int c_dtype, int64_t tiles, hipStream_t s)
{
    constexpr int W = kSpWaves;
    switch (c_dtype) {
    case TG_F32:
        hipLaunchKernelGGL((tg::gemm_sp24<tg::O_F32, CP4, W>), dim3((uint32_t)tiles), dim3(64 * W), 0, s, a);
        break;
    case TG_F16:
        hipLaunchKernelGGL((tg::gemm_sp24<tg::O_F16, CP4, W>), dim3((uint32_t)tiles), dim3(64 * W), 0, s, a);
        break;
    default:
        hipLaunchKernelGGL((tg::gemm_sp24<tg::O_BF16, CP4, W>), dim3((uint32_t)tiles), dim3(64 * W), 0, s, a);
        break;
    }
    return tg::launched();
}

}  // namespace

extern "C" tg_status tg_gemm_sp24_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                       const void* Wv, int64_t ldv, const void* Wm, int64_t ldm,
                                       void* C, int64_t ldc, tg_dtype c_dtype_arg, void* stream)
{
    const int c_dtype = tg::abi_int(c_dtype_arg);
    if (M < 0 || N < 0 || K < 0)
        return TG_ERR_INVALID_VALUE;
    if (c_dtype != TG_F32 && c_dtype != TG_F16 && c_dtype != TG_BF16)
        return TG_ERR_INVALID_VALUE;
    if (!tg::dims_fit(M, N, K, lda, ldv, ldm) || !tg::dims_fit(ldc, 0, 0))
        return TG_ERR_NOT_SUPPORTED;
    if (K % 64 != 0)
        return TG_ERR_NOT_SUPPORTED;
    if (M == 0 || N == 0)
        return TG_OK;
    if (C == nullptr || ldc < N)
        return TG_ERR_INVALID_VALUE;
    if (K > 0) {
        if (A == nullptr || Wv == nullptr || Wm == nullptr)
            return TG_ERR_INVALID_VALUE;
        if (lda < K || ldv < K / 2 || ldm < K / 8)
            return TG_ERR_INVALID_VALUE;
        if (!tg::aligned16(A) || !tg::aligned16(Wv) || ((lda * 2) & 15) || ((ldv * 2) & 15) ||
            ((uintptr_t)Wm & 3u) || (ldm & 3))
            return TG_ERR_MISALIGNED;
        if (!sp24_offsets_fit(K, lda, ldv, ldm))
            return TG_ERR_NOT_SUPPORTED;
    }
    if (!tg::aligned16(C) || ((ldc * tg::out_bytes(c_dtype)) & 15))
        return TG_ERR_MISALIGNED;
    tg::SpArgs a{M, N, K, (const uint8_t*)A, lda, (const uint8_t*)Wv, ldv, (const uint8_t*)Wm, ldm, C, ldc, 4};
    const int64_t tiles = tg::n_tiles<256, 256>(M, N);
    if (tiles > 0x7FFFFFFF)
        return TG_ERR_NOT_SUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    // codes copied once per 4 K steps where K is whole pairs of steps
    if (K % 128 == 0)
        return launch_sp24<true>(a, c_dtype, tiles, s);
    return launch_sp24<false>(a, c_dtype, tiles, s);
}
