// tg_gemm_fp8: OCP e4m3 x e4m3 -> fp32 accumulate, per-tensor scales applied
// to the accumulator before the output conversion (contract in include/tg.h).
#include <math.h>

#include "tg_host.hpp"

extern "C" tg_status tg_gemm_fp8(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, tg_layout b_layout, float scale_a,
                                 float scale_b, void* C, int64_t ldc, tg_dtype c_dtype, void* stream)
{
    bool empty;
    tg_status st = tg::check_dense(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, 1, &empty);
    if (st != TG_OK || empty)
        return st;
    if (!isfinite(scale_a) || !isfinite(scale_b))
        return TG_ERR_INVALID_VALUE;
    tg::TileArgs a{};
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
    // a row-major B (N-contiguous) goes to the generic tile kernel, which
    // transposes it on its way into LDS; the NT kernel takes the K-contiguous one
    if (b_layout == TG_COL_MAJOR)
        return tg::launch_dense<tg::E_FP8, tg::B_KCONTIG>(a, c_dtype, (hipStream_t)stream);
    return tg::launch_dense<tg::E_FP8, tg::B_NCONTIG>(a, c_dtype, (hipStream_t)stream);
}
