/*
 * CPU oracle for the tile-decomposed GEMM and the w4a16 dequant GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this file.  Only the
 * test suite, the smoke check and the bench's CPU-baseline leg use it.  It
 * shares no source with the HIP kernels.
 *
 * What it computes is the plain definition of the operation the pages build
 * their canonical kernel around:
 *
 *   C[i][j] = sum over k of A[i][k] * B[k][j]
 *
 * ("TileScale 与 TileLang比较", section 核心抽象与编程模型对比, the single-GPU
 * GEMM skeleton: a cleared register accumulator, a K loop that adds the product
 * of one A tile and one B tile per step, then one store of the accumulator.
 * Summed over all K tiles that is exactly the sum above; the tiling changes
 * only the order of the additions.)  B may be stored K x N ("row-major") or
 * N x K ("column-major", the transpose_B form used by the local GEMMs of the
 * SUMMA and Cannon examples in the "project_analysis.md" note on TileScale).
 *
 * Every element is decoded to an exact binary64 value by the scalar decoders
 * below, each product is formed in binary64 (exact: fp16 x fp16 needs 22
 * significand bits, bf16 x bf16 16, e4m3 x e4m3 8) and the products are summed
 * in k order 0..K-1 in binary64.  S[i][j] = sum of |A[i][k]|*|B[k][j]| is
 * accumulated alongside, for the acceptance bound.
 *
 * The Dequant-GEMM variant (listed as a target kernel in "TileScale 与
 * TileLang比较", sections 设计目标、定位与适用场景 and 生态互操作、性能、局限与路线图)
 * is computed in two separate steps: a scalar int4 unpack/dequant that writes
 * an fp16 weight matrix, then the dense fp16 GEMM above.  The pages give no
 * int4 format; the one used is: 8 unsigned nibbles per 32-bit word packed
 * along K, nibble j (bits 4j..4j+3) holding k = 8w + j; one fp16 scale per
 * group of `group` consecutive k per output column; a scalar zero point;
 * W = fp16_RNE((q - zero_point) * scale), rounded once.
 *
 * Threads split the output rows.  Within a row, eight output columns are
 * accumulated side by side, but each column's sum still runs in k order, so
 * the result is bit-identical to the naive triple loop (oracle_gemm_naive)
 * and independent of the thread count.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (no -ffast-math).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* element formats */
enum { ORC_F16 = 0, ORC_BF16 = 1, ORC_E4M3 = 2, ORC_F64 = 3 };
/* storage of B */
enum { ORC_B_KN = 0, ORC_B_NK = 1 };

/* ---------------------------------------------------------------- decoders */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double orc_bf16_to_f64(uint16_t b)
{
    int s = b >> 15, e = (b >> 7) & 0xFF, m = b & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);
    return s ? -v : v;
}

/* OCP fp8 e4m3 ("fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits; no
 * infinities; exponent 15 with fraction 7 is NaN; largest finite 448. */
double orc_e4m3_to_f64(uint8_t x)
{
    int s = x >> 7, e = (x >> 3) & 0xF, m = x & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* ---------------------------------------------------------------- encoders */

/* Round a finite binary64 magnitude to a binary float with `p` significand
 * bits, minimum normal exponent `emin`, round-to-nearest-even.  Returns the
 * rounded magnitude as a double (may be 2^(emax+1) on overflow: the caller
 * turns that into infinity). */
static double round_to_format(double a, int p, int emin)
{
    int ex;
    if (a == 0.0)
        return 0.0;
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) -> floor(log2 a) = ex - 1 */
    int e = ex - 1;
    if (e < emin)
        e = emin;
    double q = ldexp(1.0, e - (p - 1)); /* spacing of the format at a */
    double r = a / q;                   /* exact: division by a power of two */
    double n = nearbyint(r);            /* default mode: ties to even */
    return n * q;
}

uint16_t orc_f64_to_f16_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return 0x7E00;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7C00;
    double v = round_to_format(a, 11, -14);
    if (v == 0.0)
        return sign;
    int ex;
    frexp(v, &ex);
    int e = ex - 1;
    if (e > 15)
        return sign | 0x7C00;
    if (e < -14) /* subnormal: v = m * 2^-24 */
        return sign | (uint16_t)ldexp(v, 24);
    uint16_t m = (uint16_t)(ldexp(v, 10 - e) - 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | m;
}

uint16_t orc_f64_to_bf16_rne(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return 0x7FC0;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7F80;
    double v = round_to_format(a, 8, -126);
    if (v == 0.0)
        return sign;
    int ex;
    frexp(v, &ex);
    int e = ex - 1;
    if (e > 127)
        return sign | 0x7F80;
    if (e < -126) /* subnormal: v = m * 2^-133 */
        return sign | (uint16_t)ldexp(v, 133);
    uint16_t m = (uint16_t)(ldexp(v, 7 - e) - 128.0);
    return sign | (uint16_t)((e + 127) << 7) | m;
}

/* bulk helpers for the Python wrapper */
void orc_decode(int fmt, const void *src, double *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        switch (fmt) {
        case ORC_F16: dst[i] = orc_f16_to_f64(((const uint16_t *)src)[i]); break;
        case ORC_BF16: dst[i] = orc_bf16_to_f64(((const uint16_t *)src)[i]); break;
        case ORC_E4M3: dst[i] = orc_e4m3_to_f64(((const uint8_t *)src)[i]); break;
        default: dst[i] = ((const double *)src)[i]; break;
        }
    }
}

void orc_encode_f16(const double *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = orc_f64_to_f16_rne(src[i]);
}

void orc_encode_bf16(const double *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = orc_f64_to_bf16_rne(src[i]);
}

static double decode_one(int fmt, const void *base, int64_t idx)
{
    switch (fmt) {
    case ORC_F16: return orc_f16_to_f64(((const uint16_t *)base)[idx]);
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t *)base)[idx]);
    case ORC_E4M3: return orc_e4m3_to_f64(((const uint8_t *)base)[idx]);
    default: return ((const double *)base)[idx];
    }
}

/* ------------------------------------------------------------ int4 dequant */

/* W[n*ldw + k] = fp16_RNE((q(n,k) - zero_point) * scale(n, k/group)), with
 * q(n,k) = nibble (k mod 8) of word qweight[n*ldq + k/8].  (q - zero_point)
 * is a small integer and scale an fp16 value, so their binary64 product is
 * exact and the fp16 result is rounded exactly once. */
void orc_dequant_w4(int64_t N, int64_t K, const int32_t *qweight, int64_t ldq,
                    const uint16_t *scales, int64_t lds, int32_t group,
                    int32_t zero_point, uint16_t *W, int64_t ldw)
{
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            uint32_t word = (uint32_t)qweight[n * ldq + k / 8];
            int q = (int)((word >> (4 * (k % 8))) & 0xFu);
            double s = orc_f16_to_f64(scales[n * lds + k / group]);
            double w = (double)(q - zero_point) * s;
            W[n * ldw + k] = orc_f64_to_f16_rne(w);
        }
    }
}

/* --------------------------------------------------- 2:4 sparse weights */

/* Structured 2:4 sparsity along K of an N x K weight matrix (the sparse
 * GEMM T.gemm_sp that "TileScale 与 TileLang比较" lists in its timeline of
 * TileLang features; the page gives no storage format, so this one is a
 * reading): every aligned group of 4 consecutive k of a row keeps at most 2
 * entries.  Row n is stored as
 *   vals[n*ldv + 2g], vals[n*ldv + 2g + 1]  -- the 2 kept values of group g,
 *   code(n, g) = (meta[n*ldm + g/2] >> (4*(g%2))) & 0xF,  i0 = code & 3,
 *   i1 = code >> 2, with i0 < i1  -- their positions k = 4g + i0, 4g + i1.
 * A group with fewer than 2 nonzero entries keeps zeros in unused slots.
 * W[n*ldw + k] receives the element bits unchanged; the other two positions
 * of each group are zero.  Returns -1 (W partly written) at the first code
 * with i0 >= i1, else 0.  K must be a multiple of 4. */
int orc_expand_sp24(int64_t N, int64_t K, const uint16_t *vals, int64_t ldv,
                    const uint8_t *meta, int64_t ldm, uint16_t *W, int64_t ldw)
{
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < K / 4; ++g) {
            int code = (meta[n * ldm + g / 2] >> (4 * (g % 2))) & 0xF;
            int i0 = code & 3, i1 = code >> 2;
            if (i0 >= i1)
                return -1;
            for (int j = 0; j < 4; ++j)
                W[n * ldw + 4 * g + j] = 0;
            W[n * ldw + 4 * g + i0] = vals[n * ldv + 2 * g];
            W[n * ldw + 4 * g + i1] = vals[n * ldv + 2 * g + 1];
        }
    }
    return 0;
}

/* ------------------------------------------------------------------- GEMM */

/* Naive triple loop straight from the stored bits, single-threaded.  The
 * threaded oracle_gemm below must agree with it bit for bit. */
void orc_gemm_naive(int fmt, int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda, const void *B, int64_t ldb,
                    int b_layout, double scale_a, double scale_b,
                    double *C, double *S, int64_t ldc)
{
    double sab = scale_a * scale_b;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = decode_one(fmt, A, i * lda + k);
                double b = decode_one(fmt, B, b_layout == ORC_B_KN ? k * ldb + j : j * ldb + k);
                acc += a * b;
                mag += fabs(a) * fabs(b);
            }
            C[i * ldc + j] = acc * sab;
            if (S)
                S[i * ldc + j] = mag * fabs(sab);
        }
    }
}

struct gemm_job {
    const double *Ad; /* M x K row-major, decoded */
    const double *Bd; /* K x N row-major, decoded */
    int64_t M, N, K;
    double sab;
    double *C, *S;
    int64_t ldc;
    int64_t row0, row1;
};

#define JB 8

static void *gemm_rows(void *arg)
{
    struct gemm_job *jb = (struct gemm_job *)arg;
    const int64_t N = jb->N, K = jb->K;
    for (int64_t i = jb->row0; i < jb->row1; ++i) {
        const double *a_row = jb->Ad + i * K;
        int64_t j = 0;
        for (; j + JB <= N; j += JB) {
            double acc[JB], mag[JB];
            for (int t = 0; t < JB; ++t)
                acc[t] = mag[t] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = a_row[k];
                double aa = fabs(a);
                const double *b = jb->Bd + k * N + j;
                for (int t = 0; t < JB; ++t) {
                    acc[t] += a * b[t];
                    mag[t] += aa * fabs(b[t]);
                }
            }
            for (int t = 0; t < JB; ++t) {
                jb->C[i * jb->ldc + j + t] = acc[t] * jb->sab;
                if (jb->S)
                    jb->S[i * jb->ldc + j + t] = mag[t] * fabs(jb->sab);
            }
        }
        for (; j < N; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = a_row[k], b = jb->Bd[k * N + j];
                acc += a * b;
                mag += fabs(a) * fabs(b);
            }
            jb->C[i * jb->ldc + j] = acc * jb->sab;
            if (jb->S)
                jb->S[i * jb->ldc + j] = mag * fabs(jb->sab);
        }
    }
    return NULL;
}

/* C[i*ldc + j] = scale_a*scale_b * sum_k A[i][k]*B[k][j] (binary64), S likewise
 * with magnitudes.  A is M x K row-major with leading dimension lda; B is K x N
 * (b_layout 0, element (k,j) at k*ldb + j) or N x K (b_layout 1, element (k,j)
 * at j*ldb + k).  Returns 0 on success, -1 if memory runs out. */
int orc_gemm(int fmt, int64_t M, int64_t N, int64_t K,
             const void *A, int64_t lda, const void *B, int64_t ldb,
             int b_layout, double scale_a, double scale_b,
             double *C, double *S, int64_t ldc, int nthreads)
{
    if (M <= 0 || N <= 0)
        return 0;
    double *Ad = (double *)malloc(sizeof(double) * (size_t)(M * (K > 0 ? K : 1)));
    double *Bd = (double *)malloc(sizeof(double) * (size_t)((K > 0 ? K : 1) * N));
    if (!Ad || !Bd) {
        free(Ad);
        free(Bd);
        return -1;
    }
    for (int64_t i = 0; i < M; ++i)
        for (int64_t k = 0; k < K; ++k)
            Ad[i * K + k] = decode_one(fmt, A, i * lda + k);
    for (int64_t k = 0; k < K; ++k)
        for (int64_t j = 0; j < N; ++j)
            Bd[k * N + j] = decode_one(fmt, B, b_layout == ORC_B_KN ? k * ldb + j : j * ldb + k);

    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > M)
        nthreads = (int)M;
    struct gemm_job *jobs = (struct gemm_job *)calloc((size_t)nthreads, sizeof(struct gemm_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    int rc = 0;
    if (!jobs || !tid) {
        rc = -1;
        goto out;
    }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (struct gemm_job){Ad, Bd, M, N, K, scale_a * scale_b, C, S, ldc,
                                    M * t / nthreads, M * (t + 1) / nthreads};
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, gemm_rows, &jobs[t]) != 0)
            break;
        started = t;
    }
    gemm_rows(&jobs[0]);
    for (int t = 1; t <= started; ++t)
        pthread_join(tid[t], NULL);
    /* rows of threads that failed to start are done here */
    for (int t = started + 1; t < nthreads; ++t)
        gemm_rows(&jobs[t]);
out:
    free(jobs);
    free(tid);
    free(Ad);
    free(Bd);
    return rc;
}
