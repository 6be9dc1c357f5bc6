// tg_gemm_f16: fp16 x fp16 -> fp32 accumulate (contract in include/tg.h).
#include "tg_host.hpp"

extern "C" tg_status tg_gemm_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, tg_layout b_layout, void* C,
                                 int64_t ldc, tg_dtype c_dtype, void* stream)
{
    return tg::gemm_16bit<tg::E_F16>(M, N, K, A, lda, B, ldb, tg::abi_int(b_layout), C, ldc,
                                     tg::abi_int(c_dtype), stream);
}

// the same with a split workspace (tg_gemm_ex): instantiated here, once
tg_status tg::gemm_f16_ws(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                          int64_t ldb, int b_layout, void* C, int64_t ldc, int c_dtype, void* stream, void* ws,
                          int64_t ws_bytes)
{
    return tg::gemm_16bit<tg::E_F16>(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, stream, ws, ws_bytes);
}

int64_t tg::ws_bytes_f16(int64_t M, int64_t N, int64_t K, int b_layout)
{
    return tg::dense_ws_bytes<tg::E_F16>(M, N, K, b_layout);
}
