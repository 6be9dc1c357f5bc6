// Sanitizer driver for the host side of libtg (argument validation and the
// workspace planners), built by tests/test_sanitizers.py from the csrc/*.hip
// sources compiled for the host only, with -fsanitize=address,undefined on
// the host pass.  No call here reaches the GPU: every argument set fails
// validation, is an empty problem, or is a workspace-size query, so this runs
// on a machine without one.  The expected codes are those of include/tg.h.
// Prints "ok" and exits 0 on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include "tg.h"

static int fails = 0;
#define EXPECT(call, want)                                                                       \
    do {                                                                                         \
        const long long got_ = (long long)(call);                                                \
        if (got_ != (long long)(want)) {                                                         \
            std::fprintf(stderr, "FAIL line %d: %s = %lld, want %lld\n", __LINE__, #call, got_, \
                         (long long)(want));                                                     \
            ++fails;                                                                             \
        }                                                                                        \
    } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static const uintptr_t D = 1u << 20;  // a fake, 1 MiB aligned device address (never dereferenced)

static tg_status dense(bool bf16, int64_t M = 8, int64_t N = 8, int64_t K = 8, uintptr_t A = D, int64_t lda = 8,
                       uintptr_t B = D, int64_t ldb = 8, int lay = 0, uintptr_t C = D, int64_t ldc = 8, int cd = 0)
{
    auto f = bf16 ? tg_gemm_bf16 : tg_gemm_f16;
    return f(M, N, K, P(A), lda, P(B), ldb, (tg_layout)lay, P(C), ldc, (tg_dtype)cd, nullptr);
}

static void dense_checks()
{
    for (int t = 0; t < 2; ++t) {
        const bool b = t == 1;
        EXPECT(dense(b, -1), TG_ERR_INVALID_VALUE);
        EXPECT(dense(b, 8, 8, -3), TG_ERR_INVALID_VALUE);
        EXPECT(dense(b, 8, 8, 8, D, 8, D, 8, 2), TG_ERR_INVALID_VALUE);
        EXPECT(dense(b, 8, 8, 8, D, 8, D, 8, 0, D, 8, 7), TG_ERR_INVALID_VALUE);
        EXPECT(dense(b, 8, 8, 8, 0), TG_ERR_INVALID_VALUE);
        EXPECT(dense(b, 8, 8, 8, D, 7), TG_ERR_INVALID_VALUE);
        EXPECT(dense(b, 8, 16, 8, D, 8, D, 8, 0, D, 16), TG_ERR_INVALID_VALUE);
        EXPECT(dense(b, 8, 8, 4, D, 12), TG_ERR_MISALIGNED);
        EXPECT(dense(b, 8, 8, 8, D + 8), TG_ERR_MISALIGNED);
        EXPECT(dense(b, 8, 8, 8, D, 8, D, 8, 0, D + 4), TG_ERR_MISALIGNED);
        EXPECT(dense(b, 0, 8, 8, 0, 8, 0, 8, 0, 0), TG_OK);
        EXPECT(dense(b, 8, 0, 8, 0, 8, 0, 8, 0, 0), TG_OK);
        // sizes past 2^31 - 1 elements are refused before any offset is formed
        EXPECT(dense(b, INT64_MAX / 2, 8, 8, D, 8, D, 8, 0, D, 8), TG_ERR_NOT_SUPPORTED);
        EXPECT(dense(b, 8, 8, INT64_MAX / 4, D, INT64_MAX / 4, D, INT64_MAX / 4, 1, D, 8), TG_ERR_NOT_SUPPORTED);
        EXPECT(dense(b, 8, 8, 8, D, 8, D, 8, 0, D, 1ll << 31), TG_ERR_NOT_SUPPORTED);
    }
    EXPECT(tg_gemm_fp8(-1, 8, 8, P(D), 16, P(D), 16, TG_COL_MAJOR, 1.f, 1.f, P(D), 8, TG_F32, nullptr),
           TG_ERR_INVALID_VALUE);
    EXPECT(tg_gemm_fp8(8, 8, 8, P(D), 16, P(D), 16, TG_COL_MAJOR, INFINITY, 1.f, P(D), 8, TG_F32, nullptr),
           TG_ERR_INVALID_VALUE);
    EXPECT(tg_gemm_fp8(8, 8, 8, P(D), 16, P(D), 16, TG_COL_MAJOR, 1.f, NAN, P(D), 8, TG_F32, nullptr),
           TG_ERR_INVALID_VALUE);
    EXPECT(tg_gemm_fp8(8, 24, 8, P(D), 16, P(D), 24, TG_ROW_MAJOR, 1.f, 1.f, P(D), 24, TG_F32, nullptr),
           TG_ERR_MISALIGNED);
    EXPECT(tg_gemm_fp8(0, 8, 8, P(D), 16, P(D), 16, TG_COL_MAJOR, 1.f, 1.f, P(D), 8, TG_F32, nullptr), TG_OK);
}

static tg_status w4(int64_t M = 4, int64_t N = 8, int64_t K = 128, uintptr_t A = D, int64_t lda = 128,
                    uintptr_t q = D, int64_t ldq = 16, uintptr_t s = D, int64_t lds = 1, int g = 128, int zp = 8,
                    uintptr_t C = D, int64_t ldc = 8)
{
    return tg_gemm_w4a16(M, N, K, P(A), lda, (const int32_t*)P(q), ldq, P(s), lds, g, zp, P(C), ldc, nullptr);
}

static void w4_checks()
{
    EXPECT(w4(-1), TG_ERR_INVALID_VALUE);
    EXPECT(w4(4, 8, 128, D, 128, D, 16, D, 1, 64), TG_ERR_NOT_SUPPORTED);
    EXPECT(w4(4, 8, 200), TG_ERR_NOT_SUPPORTED);
    EXPECT(w4(4, 8, 128, D, 128, D, 16, D, 1, 128, 16), TG_ERR_NOT_SUPPORTED);
    EXPECT(w4(4, 8, 128, D, 128, 0), TG_ERR_INVALID_VALUE);
    EXPECT(w4(4, 8, 128, D, 128, D, 8), TG_ERR_INVALID_VALUE);
    EXPECT(w4(4, 8, 128, D, 128, D, 17), TG_ERR_MISALIGNED);
    EXPECT(w4(4, 8, 128, D, 128, D, 16, D + 1), TG_ERR_MISALIGNED);
    EXPECT(w4(4, 8, 128, D + 2), TG_ERR_MISALIGNED);
    EXPECT(w4(4, 8, 128, D, 128, D, 16, D, 1, 128, 8, D, 4), TG_ERR_INVALID_VALUE);
    EXPECT(w4(0), TG_OK);
    EXPECT(w4(INT64_MAX / 2, 8, 128, D, 128, D, 16, D, 1, 128, 8, D, 8), TG_ERR_NOT_SUPPORTED);
    EXPECT(w4(4, 8, 1ll << 40, D, 1ll << 40, D, 1ll << 37, D, 1ll << 33), TG_ERR_NOT_SUPPORTED);
    EXPECT(tg_dequant_w4(8, 128, (const int32_t*)P(D), 16, P(D), 1, 128, 8, nullptr, 128, nullptr),
           TG_ERR_INVALID_VALUE);
    EXPECT(tg_dequant_w4(8, 100, (const int32_t*)P(D), 16, P(D), 1, 128, 8, P(D), 128, nullptr),
           TG_ERR_NOT_SUPPORTED);
    EXPECT(tg_dequant_w4(0, 128, nullptr, 16, nullptr, 1, 128, 8, nullptr, 128, nullptr), TG_OK);
    const int64_t need = tg_gemm_w4a16_ex_workspace_bytes(256, 8192, 8192);
    EXPECT(need > 65536, 1);
    EXPECT(tg_gemm_w4a16_ex(256, 8192, 8192, P(D), 8192, (const int32_t*)P(D), 1024, P(D), 64, 128, 8, P(D), 8192,
                            P(D), need - 1, nullptr),
           TG_ERR_INVALID_VALUE);
    EXPECT(tg_gemm_w4a16_ex(256, 8192, 8192, P(D), 8192, (const int32_t*)P(D), 1024, P(D), 64, 128, 8, P(D), 8192,
                            P(D + 64), need, nullptr),
           TG_ERR_MISALIGNED);
}

static void sp24_checks()
{
    auto call = [](int64_t M, int64_t K, uintptr_t A, int64_t lda, int64_t ldm, int dt) {
        return tg_gemm_sp24_bf16(M, 64, K, P(A), lda, P(D), 64, P(D), ldm, P(D), 64, (tg_dtype)dt, nullptr);
    };
    EXPECT(call(-1, 128, D, 128, 16, 2), TG_ERR_INVALID_VALUE);
    EXPECT(call(64, 96, D, 128, 16, 2), TG_ERR_NOT_SUPPORTED);
    EXPECT(call(64, 128, D, 128, 16, 7), TG_ERR_INVALID_VALUE);
    EXPECT(call(64, 128, D + 2, 128, 16, 2), TG_ERR_MISALIGNED);
    EXPECT(call(64, 128, D, 128, 15, 2), TG_ERR_INVALID_VALUE);
    EXPECT(call(64, 128, D, 1 << 30, 16, 2), TG_ERR_NOT_SUPPORTED);
    EXPECT(call(0, 128, D, 128, 16, 2), TG_OK);
}

static void ex_checks()
{
    static const int64_t sizes[] = {0,     1,     7,       16,         33,         64,        255,
                                    256,   4096,  8192,    12345,      65536,      1 << 20,   0x7FFFFFFF,
                                    1ll << 31, 1ll << 40, INT64_MAX / 3, INT64_MAX};
    // the planners over every combination: a size or -1, never UB
    for (int in = -1; in <= 3; ++in)
        for (int lay = 0; lay < 2; ++lay)
            for (int64_t M : sizes)
                for (int64_t N : sizes)
                    for (int64_t K : sizes) {
                        const int64_t b = tg_gemm_ex_workspace_bytes((tg_input)in, M, N, K, (tg_layout)lay);
                        EXPECT(b >= (in >= 0 && in <= 2 ? 0 : -1), 1);
                        if (in == 0 && lay == 0) {
                            const int64_t w = tg_gemm_w4a16_ex_workspace_bytes(M, N, K);
                            EXPECT(w >= 0, 1);
                        }
                    }
    EXPECT(tg_gemm_ex_workspace_bytes(TG_IN_BF16, -1, 8, 8, TG_COL_MAJOR), -1);
    EXPECT(tg_gemm_w4a16_ex_workspace_bytes(-1, 8, 128), -1);
    const int64_t need = tg_gemm_ex_workspace_bytes(TG_IN_BF16, 256, 8192, 8192, TG_COL_MAJOR);
    EXPECT(need > 65536, 1);
    auto call = [](int in, int64_t M, int64_t lda, uintptr_t ws, int64_t nbytes) {
        return tg_gemm_ex((tg_input)in, M, 8192, 8192, P(D), lda, P(D), 8192, TG_COL_MAJOR, 1.f, 1.f, P(D), 8192,
                          TG_BF16, P(ws), nbytes, nullptr);
    };
    EXPECT(call(5, 256, 8192, D, 1 << 30), TG_ERR_INVALID_VALUE);
    EXPECT(call(1, 256, 8192, D, -1), TG_ERR_INVALID_VALUE);
    EXPECT(call(1, 256, 8192, 0, 256), TG_ERR_INVALID_VALUE);
    EXPECT(call(1, 256, 8192, D, need - 1), TG_ERR_INVALID_VALUE);
    EXPECT(call(1, 256, 8192, D + 16, 1 << 30), TG_ERR_MISALIGNED);
    EXPECT(call(1, 256, 8, D, 1 << 30), TG_ERR_INVALID_VALUE);
    EXPECT(call(1, 0, 8192, D, 1 << 30), TG_OK);
    auto na = [](int in, int64_t M, uintptr_t C, int cd, float sa) {
        return tg_gemm_ex_noalloc((tg_input)in, M, 8192, 8192, P(D), 8192, P(D), 8192, TG_COL_MAJOR, sa, 1.f, P(C),
                                  8192, (tg_dtype)cd, nullptr);
    };
    EXPECT(na(9, 256, D, 2, 1.f), TG_ERR_INVALID_VALUE);
    EXPECT(na(1, -1, D, 2, 1.f), TG_ERR_INVALID_VALUE);
    EXPECT(na(1, 256, D + 2, 2, 1.f), TG_ERR_MISALIGNED);
    EXPECT(na(2, 256, D, 2, NAN), TG_ERR_INVALID_VALUE);
    EXPECT(na(1, 0, D, 2, 1.f), TG_OK);
}

int main()
{
    for (int s = -2; s <= 8; ++s)
        if (tg_status_string((tg_status)s) == nullptr || std::strlen(tg_status_string((tg_status)s)) == 0)
            ++fails;
    EXPECT(tg_version() > 0, 1);
    dense_checks();
    w4_checks();
    sp24_checks();
    ex_checks();
    if (fails) {
        std::fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    std::puts("ok");
    return 0;
}
