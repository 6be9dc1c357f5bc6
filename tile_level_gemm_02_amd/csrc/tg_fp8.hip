// tg_gemm_fp8: OCP e4m3 x e4m3 -> fp32 accumulate, per-tensor scales applied
// to the accumulator before the output conversion (contract in include/tg.h).
// Both layouts of B run the NT kernel where its element grid and tile sizes
// allow (a row-major B through transposing LDS reads), else the generic
// tile kernel (gemm_fp8 in tg_host.hpp).
#include "tg_host.hpp"

extern "C" tg_status tg_gemm_fp8(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, tg_layout b_layout, float scale_a,
                                 float scale_b, void* C, int64_t ldc, tg_dtype c_dtype, void* stream)
{
    return tg::gemm_fp8(M, N, K, A, lda, B, ldb, tg::abi_int(b_layout), scale_a, scale_b, C, ldc, tg::abi_int(c_dtype),
                        stream);
}

// the same with a split workspace (tg_gemm_ex): instantiated here, once
tg_status tg::gemm_fp8_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                          int b_layout, float scale_a, float scale_b, void* C, int64_t ldc, int c_dtype, void* stream,
                          void* ws, int64_t ws_bytes)
{
    return tg::gemm_fp8(M, N, K, A, lda, B, ldb, b_layout, scale_a, scale_b, C, ldc, c_dtype, stream, ws, ws_bytes);
}

int64_t tg::ws_bytes_fp8(int64_t M, int64_t N, int64_t K, int b_layout)
{
    return tg::dense_ws_bytes<tg::E_FP8>(M, N, K, b_layout);
}
