/* Sanitizer driver for oracle/oracle.c (built with -fsanitize=address,undefined
 * by tests/test_sanitizers.py).  Every buffer is allocated at its exact extent
 * (last element + 1), so a read or write one element past what a function may
 * touch is reported.  Checks, besides the sanitizers' own: the codecs round-trip
 * every finite 16-bit pattern, the threaded GEMM equals the naive triple loop
 * bit for bit at every thread count, and the sp24 expander rejects a bad code.
 * Prints "ok" and exits 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_f16_to_f64(uint16_t h);
double orc_bf16_to_f64(uint16_t b);
double orc_e4m3_to_f64(uint8_t x);
uint16_t orc_f64_to_f16_rne(double x);
uint16_t orc_f64_to_bf16_rne(double x);
void orc_decode(int fmt, const void *src, double *dst, int64_t n);
void orc_dequant_w4(int64_t N, int64_t K, const int32_t *qweight, int64_t ldq, const uint16_t *scales,
                    int64_t lds, int32_t group, int32_t zero_point, uint16_t *W, int64_t ldw);
int orc_expand_sp24(int64_t N, int64_t K, const uint16_t *vals, int64_t ldv, const uint8_t *meta, int64_t ldm,
                    uint16_t *W, int64_t ldw);
void orc_gemm_naive(int fmt, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
                    int64_t ldb, int b_layout, double scale_a, double scale_b, double *C, double *S, int64_t ldc);
int orc_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
             int b_layout, double scale_a, double scale_b, double *C, double *S, int64_t ldc, int nthreads);

static int fails = 0;
#define CHECK(c, ...)                                   \
    do {                                                \
        if (!(c)) {                                     \
            fprintf(stderr, "FAIL %s:%d ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);               \
            fputc('\n', stderr);                        \
            ++fails;                                    \
        }                                               \
    } while (0)

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 16);
}

/* exact extent of a rows x cols matrix with leading dimension ld (0 if empty) */
static size_t extent(int64_t rows, int64_t cols, int64_t ld)
{
    return rows > 0 && cols > 0 ? (size_t)((rows - 1) * ld + cols) : 0;
}

static void *xmalloc(size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* random finite element bits of format fmt (0 f16, 1 bf16, 2 e4m3, 3 f64) */
static void fill(int fmt, void *p, size_t n)
{
    for (size_t i = 0; i < n; ++i) {
        if (fmt == 0) {
            uint16_t h;
            do h = (uint16_t)next32(); while (((h >> 10) & 0x1F) == 0x1F);
            ((uint16_t *)p)[i] = h;
        } else if (fmt == 1) {
            uint16_t b;
            do b = (uint16_t)next32(); while (((b >> 7) & 0xFF) == 0xFF);
            ((uint16_t *)p)[i] = b;
        } else if (fmt == 2) {
            uint8_t x;
            do x = (uint8_t)next32(); while ((x & 0x7F) == 0x7F);
            ((uint8_t *)p)[i] = x;
        } else {
            ((double *)p)[i] = ldexp((double)(int32_t)next32(), -31);
        }
    }
}

static void codecs(void)
{
    for (uint32_t h = 0; h < 65536; ++h) {
        double x = orc_f16_to_f64((uint16_t)h);
        if (!isnan(x))
            CHECK(orc_f64_to_f16_rne(x) == h, "f16 round trip of 0x%04x", h);
        double y = orc_bf16_to_f64((uint16_t)h);
        if (!isnan(y))
            CHECK(orc_f64_to_bf16_rne(y) == h, "bf16 round trip of 0x%04x", h);
    }
    for (uint32_t v = 0; v < 256; ++v) {
        double e = orc_e4m3_to_f64((uint8_t)v);
        CHECK(isnan(e) == ((v & 0x7F) == 0x7F), "e4m3 NaN pattern 0x%02x", v);
    }
    uint16_t src[7];
    double dst[7];
    fill(0, src, 7);
    orc_decode(0, src, dst, 7);
    for (int i = 0; i < 7; ++i)
        CHECK(dst[i] == orc_f16_to_f64(src[i]), "decode element %d", i);
}

static void gemm_case(int fmt, int64_t M, int64_t N, int64_t K, int lay, int pad)
{
    static const size_t item[4] = {2, 2, 1, 8};
    const int64_t lda = K + pad, ldb = (lay == 0 ? N : K) + pad, ldc = N + pad;
    const size_t na = extent(M, K, lda), nb = lay == 0 ? extent(K, N, ldb) : extent(N, K, ldb);
    const size_t nc = extent(M, N, ldc);
    void *A = xmalloc(na * item[fmt]), *B = xmalloc(nb * item[fmt]);
    double *C1 = (double *)xmalloc(nc * 8), *S1 = (double *)xmalloc(nc * 8);
    double *C2 = (double *)xmalloc(nc * 8), *S2 = (double *)xmalloc(nc * 8);
    fill(fmt, A, na);
    fill(fmt, B, nb);
    const double sa = fmt == 2 ? 0.75 : 1.0, sb = fmt == 2 ? -2.0 : 1.0;
    orc_gemm_naive(fmt, M, N, K, A, lda, B, ldb, lay, sa, sb, C1, S1, ldc);
    for (int t = 1; t <= 5; t += 2) {
        memset(C2, 0, nc * 8);
        memset(S2, 0, nc * 8);
        CHECK(orc_gemm(fmt, M, N, K, A, lda, B, ldb, lay, sa, sb, C2, S2, ldc, t) == 0, "orc_gemm status");
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                const size_t x = (size_t)(i * ldc + j);
                CHECK(memcmp(&C1[x], &C2[x], 8) == 0 && memcmp(&S1[x], &S2[x], 8) == 0,
                      "fmt %d %lldx%lldx%lld lay %d threads %d at (%lld,%lld)", fmt, (long long)M, (long long)N,
                      (long long)K, lay, t, (long long)i, (long long)j);
            }
    }
    free(A);
    free(B);
    free(C1);
    free(S1);
    free(C2);
    free(S2);
}

static void dequant(void)
{
    const int64_t N = 5, K = 256, ldq = K / 8 + 3, lds = K / 128 + 1, ldw = K + 5;
    int32_t *q = (int32_t *)xmalloc(extent(N, K / 8, ldq) * 4);
    uint16_t *s = (uint16_t *)xmalloc(extent(N, K / 128, lds) * 2);
    uint16_t *W = (uint16_t *)xmalloc(extent(N, K, ldw) * 2);
    for (size_t i = 0; i < extent(N, K / 8, ldq); ++i)
        q[i] = (int32_t)next32();
    fill(0, s, extent(N, K / 128, lds));
    for (int zp = 0; zp <= 15; zp += 5) {
        orc_dequant_w4(N, K, q, ldq, s, lds, 128, zp, W, ldw);
        for (int64_t n = 0; n < N; ++n)
            for (int64_t k = 0; k < K; k += 37) {
                const int nib = (int)(((uint32_t)q[n * ldq + k / 8] >> (4 * (k % 8))) & 15u);
                const double ref = (nib - zp) * orc_f16_to_f64(s[n * lds + k / 128]);
                CHECK(W[n * ldw + k] == orc_f64_to_f16_rne(ref), "dequant (%lld,%lld)", (long long)n, (long long)k);
            }
    }
    free(q);
    free(s);
    free(W);
}

static void sp24(void)
{
    const int64_t N = 3, K = 64, ldv = K / 2 + 2, ldm = K / 8 + 1, ldw = K + 3;
    static const uint8_t codes[6] = {0x4, 0x8, 0xC, 0x9, 0xD, 0xE}; /* every i0 < i1 */
    uint16_t *v = (uint16_t *)xmalloc(extent(N, K / 2, ldv) * 2);
    uint8_t *m = (uint8_t *)xmalloc(extent(N, K / 8, ldm));
    uint16_t *W = (uint16_t *)xmalloc(extent(N, K, ldw) * 2);
    fill(1, v, extent(N, K / 2, ldv));
    for (size_t i = 0; i < extent(N, K / 8, ldm); ++i)
        m[i] = (uint8_t)(codes[next32() % 6] | (codes[next32() % 6] << 4));
    CHECK(orc_expand_sp24(N, K, v, ldv, m, ldm, W, ldw) == 0, "valid codes rejected");
    m[ldm + 1] = 0x11; /* i0 == i1 in row 1 */
    CHECK(orc_expand_sp24(N, K, v, ldv, m, ldm, W, ldw) == -1, "bad code accepted");
    free(v);
    free(m);
    free(W);
}

int main(void)
{
    static const int64_t shapes[][3] = {{0, 3, 4}, {3, 0, 4}, {2, 3, 0}, {1, 1, 1}, {5, 9, 13},
                                        {17, 8, 33}, {9, 17, 64}};
    codecs();
    for (int fmt = 0; fmt < 4; ++fmt)
        for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
            for (int lay = 0; lay < 2; ++lay)
                for (int pad = 0; pad < 2; ++pad)
                    gemm_case(fmt, shapes[s][0], shapes[s][1], shapes[s][2], lay, 3 * pad);
    dequant();
    sp24();
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    puts("ok");
    return 0;
}
