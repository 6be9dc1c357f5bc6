// tg_gemm_f16: fp16 x fp16 -> fp32 accumulate (contract in include/tg.h).
#include "tg_host.hpp"

extern "C" tg_status tg_gemm_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, tg_layout b_layout, void* C,
                                 int64_t ldc, tg_dtype c_dtype, void* stream)
{
    return tg::gemm_16bit<tg::E_F16>(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, stream);
}
