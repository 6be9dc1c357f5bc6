// tg_gemm_ex_noalloc: tg_gemm_ex for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation), with the split workspace in a static device array of
// this library instead of a caller buffer (contract in include/tg.h).
#include <mutex>

#include "tg_host.hpp"

namespace tg {
int64_t ex_workspace_bytes(int in, int64_t M, int64_t N, int64_t K, int b_layout);  // tg_ex.hip
}

namespace {

// The scratch: every split plan the library makes needs at most 64 KiB of
// arrival counters plus 64 MiB of partial tiles (one round of at most 256
// split workgroups, each with a partial tile of at most 256 x 256 fp32), so
// that is its size.  Each GPU holds its own copy, at its own address, until the
// process ends.
constexpr int64_t kScratchBytes = (64 << 20) + (64 << 10);
constexpr int64_t kScratchCounterWords = (64 << 10) / 4;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Zero the counter words (a kernel, so that a captured call records no memset).
__global__ __launch_bounds__(256) void zero_counters(uint32_t* p, int64_t words)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < words)
        p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (set up once)

// Device address of this device's scratch, looked up (and its counters
// cleared, on `stream`) on the first call made with the device current.
tg_status scratch_of_current_device(hipStream_t stream, void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TG_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
            return TG_ERR_LAUNCH;
        hipLaunchKernelGGL(zero_counters, dim3((uint32_t)((kScratchCounterWords + 255) / 256)), dim3(256), 0, stream,
                           (uint32_t*)ptr, kScratchCounterWords);
        if (hipGetLastError() != hipSuccess)
            return TG_ERR_LAUNCH;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return TG_OK;
}

}  // namespace

extern "C" tg_status tg_gemm_ex_noalloc(tg_input in_arg, int64_t M, int64_t N, int64_t K, const void* A,
                                        int64_t lda, const void* B, int64_t ldb, tg_layout b_layout_arg, float scale_a,
                                        float scale_b, void* C, int64_t ldc, tg_dtype c_dtype_arg, void* stream)
{
    const int in = tg::abi_int(in_arg), b_layout = tg::abi_int(b_layout_arg), c_dtype = tg::abi_int(c_dtype_arg);
    if (in != TG_IN_F16 && in != TG_IN_BF16 && in != TG_IN_FP8)
        return TG_ERR_INVALID_VALUE;
    // every argument is checked before the first HIP call (the scratch set-up)
    bool empty;
    const tg_status chk = tg::check_dense(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, in == TG_IN_FP8 ? 1 : 2,
                                          &empty);
    if (chk != TG_OK || empty)
        return chk;
    if (in == TG_IN_FP8 && (!__builtin_isfinite(scale_a) || !__builtin_isfinite(scale_b)))
        return TG_ERR_INVALID_VALUE;
    const int64_t need = tg::ex_workspace_bytes(in, M, N, K, b_layout);
    if (need < 0)
        return TG_ERR_INVALID_VALUE;
    if (need > kScratchBytes)
        return TG_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        const tg_status st = scratch_of_current_device((hipStream_t)stream, &ws);
        if (st != TG_OK)
            return st;
    }
    const int64_t ws_bytes = ws != nullptr ? kScratchBytes : 0;
    switch (in) {
    case TG_IN_F16:
        return tg::gemm_f16_ws(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, stream, ws, ws_bytes);
    case TG_IN_BF16:
        return tg::gemm_bf16_ws(M, N, K, A, lda, B, ldb, b_layout, C, ldc, c_dtype, stream, ws, ws_bytes);
    default:
        return tg::gemm_fp8_ws(M, N, K, A, lda, B, ldb, b_layout, scale_a, scale_b, C, ldc, c_dtype, stream, ws,
                               ws_bytes);
    }
}
