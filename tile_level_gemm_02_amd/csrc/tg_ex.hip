// tg_gemm_ex and tg_gemm_ex_workspace_bytes: the dense GEMM of every input
// type with a caller workspace, which lets the NT kernel split K over
// several workgroups per output tile (contract in include/tg.h).
#include "tg_abi.hpp"

namespace tg {
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

// tg_gemm_ex_workspace_bytes on the int values of its enum arguments
int64_t ex_workspace_bytes(int in, int64_t M, int64_t N, int64_t K, int b_layout)
{
    if (M < 0 || N < 0 || K < 0 || (b_layout != TG_ROW_MAJOR && b_layout != TG_COL_MAJOR))
        return -1;
    switch (in) {
    case TG_IN_F16: return ws_bytes_f16(M, N, K, b_layout);
    case TG_IN_BF16: return ws_bytes_bf16(M, N, K, b_layout);
    case TG_IN_FP8: return ws_bytes_fp8(M, N, K, b_layout);
    default: return -1;
    }
}
}  // namespace tg

extern "C" int64_t tg_gemm_ex_workspace_bytes(tg_input in_arg, int64_t M, int64_t N, int64_t K,
                                              tg_layout b_layout_arg)
{
    return tg::ex_workspace_bytes(tg::abi_int(in_arg), M, N, K, tg::abi_int(b_layout_arg));
}

extern "C" tg_status tg_gemm_ex(tg_input in_arg, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                const void* B, int64_t ldb, tg_layout b_layout_arg, float scale_a, float scale_b,
                                void* C, int64_t ldc, tg_dtype c_dtype_arg, void* workspace, int64_t workspace_bytes,
                                void* stream)
{
    const int in = tg::abi_int(in_arg), b_layout = tg::abi_int(b_layout_arg), c_dtype = tg::abi_int(c_dtype_arg);
    if (in != TG_IN_F16 && in != TG_IN_BF16 && in != TG_IN_FP8)
        return TG_ERR_INVALID_VALUE;
    if (workspace_bytes < 0 || (workspace == nullptr && workspace_bytes != 0))
        return TG_ERR_INVALID_VALUE;
    if (workspace != nullptr) {
        if (((uintptr_t)workspace & 255u) != 0)
            return TG_ERR_MISALIGNED;
        const int64_t need = tg::ex_workspace_bytes(in, M, N, K, b_layout);
        if (need < 0)
            return TG_ERR_INVALID_VALUE;
        if (workspace_bytes < need)
            return TG_ERR_INVALID_VALUE;
    }
    switch (in) {
    case TG_IN_F16:
        return tg::gemm_f16_ws(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, stream, workspace, workspace_bytes);
    case TG_IN_BF16:
        return tg::gemm_bf16_ws(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, stream, workspace, workspace_bytes);
    default:
        return tg::gemm_fp8_ws(M, N, K, A, lda, B, ldb, b_layout, scale_a, scale_b, C, ldc, c_dtype, stream, workspace,
                               workspace_bytes);
    }
}
