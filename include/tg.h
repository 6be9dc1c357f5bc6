/*
 * tg.h -- C ABI of the tile GEMM library for AMD MI355X (gfx950).
 *
 * The library computes the tile-decomposed matrix multiply C = A.B that
 * TileLang and TileScale use as their canonical kernel, its weight-only
 * int4 "Dequant-GEMM" variant and a 2:4 structured-sparse variant.
 * Operation, per call:
 *
 *     C[i][j] = alpha * sum over k of A[i][k] * B[k][j]      (fp32 accumulate)
 *
 * with alpha = 1 except for the fp8 entry point (alpha = scale_a * scale_b).
 * Source of the operation: the single-GPU GEMM skeleton of "TileScale 与
 * TileLang比较" (yaopepe.com), section 核心抽象与编程模型对比 -- an output-tile
 * grid, shared-memory tiles of A and B, a cleared register accumulator, a
 * pipelined loop over K that adds one tile product per step, and a final store
 * of the accumulator.  Sizes need not divide the tile (the TileScale README's
 * GEMM example sizes its grid with ceildiv).  The Dequant-GEMM is named as a
 * target kernel in the same page, sections 设计目标、定位与适用场景 and
 * 生态互操作、性能、局限与路线图.
 *
 * Conventions shared by every entry point
 *  - Pointers A, B, C, qweight, scales, W, Wv, Wm, workspace are DEVICE
 *    pointers owned by the caller.  The library never allocates, frees or
 *    retains them and keeps no state between calls (it is reentrant).
 *  - Matrices are row-major with a leading dimension in ELEMENTS:
 *      A      : M x K, element (i,k) at A[i*lda + k], lda >= K
 *      B      : TG_ROW_MAJOR: K x N, element (k,j) at B[k*ldb + j], ldb >= N
 *               TG_COL_MAJOR: stored N x K, element (k,j) at B[j*ldb + k], ldb >= K
 *               (the transpose_B form; the layout of an nn.Linear weight)
 *      C      : M x N, element (i,j) at C[i*ldc + j], ldc >= N
 *  - C is overwritten (no beta).  M == 0 or N == 0 is a no-op returning TG_OK.
 *    K == 0 stores zeros (an empty sum).  Any M, N, K >= 1 is handled; tails
 *    that do not fill a tile are masked.
 *  - Alignment: every base pointer 16-byte aligned and every leading dimension
 *    times the element size a multiple of 16 bytes; else TG_ERR_MISALIGNED.
 *  - C must not overlap A or B (not checked).
 *  - Execution is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream).  No call synchronizes.  Argument validation is synchronous and
 *    happens before any HIP call: an invalid call launches nothing.  A failed
 *    launch returns TG_ERR_LAUNCH.  Faults inside a kernel surface at the
 *    caller's next synchronization.
 *  - Sizes are int64; leading dimensions and sizes must be non-negative and
 *    every index must fit in the addressed buffer (the caller's duty).  A
 *    size or leading dimension above 2^31 - 1 elements returns
 *    TG_ERR_NOT_SUPPORTED (the workspace queries report 0 for such shapes).
 *  - Enum arguments are read as the int the C ABI passes: any int is
 *    accepted, and a value that names no enumerator is TG_ERR_INVALID_VALUE.
 */
#ifndef TG_H
#define TG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TG_OK = 0,
    TG_ERR_INVALID_VALUE = 1, /* negative size, ld too small, NULL pointer, bad enum */
    TG_ERR_NOT_SUPPORTED = 2, /* valid request the library does not implement */
    TG_ERR_MISALIGNED = 3,    /* base pointer or leading dimension not 16-byte aligned */
    TG_ERR_LAUNCH = 4,        /* the HIP runtime refused the launch */
    TG_ERR_SCRATCH = 5        /* the problem needs more scratch than tg_gemm_ex_noalloc's static buffer */
} tg_status;

typedef enum { TG_F32 = 0, TG_F16 = 1, TG_BF16 = 2 } tg_dtype;

/* storage of B (a K x N operand) */
typedef enum { TG_ROW_MAJOR = 0, TG_COL_MAJOR = 1 } tg_layout;

/* fp16 x fp16 -> fp32 accumulate -> C of c_dtype (TG_F32, TG_F16 or TG_BF16;
 * conversion is round-to-nearest-even).  A, B hold IEEE binary16 elements. */
tg_status tg_gemm_f16(int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t lda,
                      const void *B, int64_t ldb, tg_layout b_layout,
                      void *C, int64_t ldc, tg_dtype c_dtype,
                      void *stream);

/* bf16 x bf16 -> fp32 accumulate -> C of c_dtype.  Same contract as
 * tg_gemm_f16 with bfloat16 inputs. */
tg_status tg_gemm_bf16(int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda,
                       const void *B, int64_t ldb, tg_layout b_layout,
                       void *C, int64_t ldc, tg_dtype c_dtype,
                       void *stream);

/* fp8 (OCP e4m3, "e4m3fn": bias 7, max 448, no inf) x fp8 -> fp32
 * accumulate; C = (scale_a * scale_b) * (Aq . Bq), converted to c_dtype.
 * scale_a, scale_b are per-tensor dequantisation scales passed by value
 * (finite).  Both layouts of B are taken.  With TG_ROW_MAJOR, problems of
 * at least a few hundred output tiles with N and K multiples of 16 run at
 * the speed of TG_COL_MAJOR; others run a slower kernel that transposes B
 * on its way into shared memory. */
tg_status tg_gemm_fp8(int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t lda,
                      const void *B, int64_t ldb, tg_layout b_layout,
                      float scale_a, float scale_b,
                      void *C, int64_t ldc, tg_dtype c_dtype,
                      void *stream);

/* w4a16: fp16 activations x int4 weights -> fp32 accumulate -> fp16 C.
 *   A       : fp16 M x K row-major (lda)
 *   qweight : int32 [N][ldq], ldq >= ceil(K/8); word w of row n packs
 *             k = 8w .. 8w+7, nibble j (bits 4j..4j+3) holding k = 8w + j
 *   scales  : fp16 [N][lds], lds >= ceil(K/group_size); one scale per
 *             group of group_size consecutive k of column n
 *   weight  : W[k][n] = fp16_RNE((q - zero_point) * scale[n][k/group_size]),
 *             rounded once (bit-identical to tg_dequant_w4)
 * Supported: group_size == 128, K % 128 == 0, 0 <= zero_point <= 15; other
 * values return TG_ERR_NOT_SUPPORTED.  The int4 format is not given by the
 * pages; this packing is the plain reading of "8 per int32 along K".
 * Alignment: A, qweight 16 bytes; scales 2 bytes; lda*2 and ldq*4 multiples
 * of 16; C 16 bytes with ldc*2 a multiple of 16. */
tg_status tg_gemm_w4a16(int64_t M, int64_t N, int64_t K,
                        const void *A, int64_t lda,
                        const int32_t *qweight, int64_t ldq,
                        const void *scales, int64_t lds,
                        int32_t group_size, int32_t zero_point,
                        void *C, int64_t ldc,
                        void *stream);

/* Bytes of workspace tg_gemm_w4a16_ex can use for this problem to split K
 * over several workgroups per output tile (0: it never splits this problem);
 * -1 for a negative size. */
int64_t tg_gemm_w4a16_ex_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* tg_gemm_w4a16 (same operands, formats, limits and results) with a
 * workspace that lets the library split K over several workgroups per output
 * tile where the batch has too few rows to fill the chip with its own tiles
 * (e.g. 256 rows against an 8192 x 8192 weight): a kernel with 128 x 128
 * tiles, in which each dequantised weight feeds four matrix instructions,
 * stores fp32 partial tiles in the workspace and the last workgroup of a
 * tile to finish adds them in split order (repeated calls are bit-identical)
 * and stores C.  The workspace follows the contract of tg_gemm_ex (device
 * memory, 256-byte aligned, its first 64 KiB zero before first use and left
 * zero by every call; one workspace per concurrently running call; NULL with
 * workspace_bytes 0: exactly tg_gemm_w4a16).  Errors: TG_ERR_INVALID_VALUE
 * for a negative workspace_bytes, a NULL workspace with workspace_bytes != 0
 * or a workspace smaller than tg_gemm_w4a16_ex_workspace_bytes reports;
 * TG_ERR_MISALIGNED for a workspace not 256-byte aligned; otherwise as
 * tg_gemm_w4a16. */
tg_status tg_gemm_w4a16_ex(int64_t M, int64_t N, int64_t K,
                           const void *A, int64_t lda,
                           const int32_t *qweight, int64_t ldq,
                           const void *scales, int64_t lds,
                           int32_t group_size, int32_t zero_point,
                           void *C, int64_t ldc,
                           void *workspace, int64_t workspace_bytes,
                           void *stream);

/* The dequant step of tg_gemm_w4a16 alone: writes W as fp16 [N][K] with
 * leading dimension ldw (W[n*ldw + k]), using the same device routine the
 * GEMM uses, so the two are bit-identical.  Same limits as tg_gemm_w4a16;
 * W must be 16-byte aligned with ldw*2 a multiple of 16. */
tg_status tg_dequant_w4(int64_t N, int64_t K,
                        const int32_t *qweight, int64_t ldq,
                        const void *scales, int64_t lds,
                        int32_t group_size, int32_t zero_point,
                        void *W, int64_t ldw,
                        void *stream);

/* 2:4 structured-sparse GEMM: bf16 activations x 2:4-sparse bf16 weights ->
 * fp32 accumulate -> C of c_dtype (TG_F32, TG_F16 or TG_BF16, RNE).
 *     C[i][j] = sum over k of A[i][k] * W[j][k]
 * W is N x K (the transpose_B form) with at most 2 nonzero entries in every
 * aligned group of 4 consecutive k of a row, stored compressed:
 *   Wv : bf16 [N][ldv], ldv >= K/2: the 2 kept values of group g of row n at
 *        Wv[n*ldv + 2g] and Wv[n*ldv + 2g + 1], in position order
 *   Wm : uint8 [N][ldm], ldm >= K/8: the 4-bit code of group g of row n is
 *        (Wm[n*ldm + g/2] >> (4*(g%2))) & 0xF = i0 | (i1 << 2), the positions
 *        k = 4g + i0 and 4g + i1 of the two kept values, i0 < i1 (a group
 *        with fewer nonzeros keeps zeros in its unused slots)
 * Source: the sparse GEMM T.gemm_sp in the TileLang timeline of "TileScale
 * 与 TileLang比较"; the page gives no storage format, this one is a reading
 * (the layout of the gfx950 sparse matrix instructions' index operand).  A
 * code with i0 >= i1 is outside the format: it is not checked (device data),
 * and each kept value then multiplies the activation at its coded position.
 * Supported: K % 64 == 0 (else TG_ERR_NOT_SUPPORTED).  Alignment: A, Wv, C
 * 16 bytes with lda*2, ldv*2 and ldc*element size multiples of 16; Wm 4
 * bytes with ldm a multiple of 4; else TG_ERR_MISALIGNED.  Other conventions
 * as above (Wv, Wm are device pointers). */
tg_status tg_gemm_sp24_bf16(int64_t M, int64_t N, int64_t K,
                            const void *A, int64_t lda,
                            const void *Wv, int64_t ldv,
                            const void *Wm, int64_t ldm,
                            void *C, int64_t ldc, tg_dtype c_dtype,
                            void *stream);

/* Input element type of tg_gemm_ex. */
typedef enum { TG_IN_F16 = 0, TG_IN_BF16 = 1, TG_IN_FP8 = 2 } tg_input;

/* Bytes of workspace tg_gemm_ex can use for this problem to split its K
 * range over several workgroups per output tile (0: it never splits this
 * problem, a NULL workspace is then as good as any); -1 for a negative size
 * or an invalid enum.  Depends only on the arguments given (not on leading
 * dimensions or output type), so it may be queried once per shape. */
int64_t tg_gemm_ex_workspace_bytes(tg_input in, int64_t M, int64_t N, int64_t K,
                                   tg_layout b_layout);

/* The dense GEMM of tg_gemm_f16 / tg_gemm_bf16 / tg_gemm_fp8 (selected by
 * `in`; same operands, layouts, conventions and results) with a workspace
 * that lets the library split K over several workgroups per output tile
 * where too few output tiles would leave the chip's compute units idle or
 * re-read the operands too often (e.g. a few hundred rows against an
 * 8192 x 8192 weight), or where the output tiles take more than one round
 * of the chip and the last round is short (e.g. 4608 x 4608: 324 tiles of
 * 256 x 256 on 256 compute units): the full rounds then run whole tiles and
 * only the last round's tiles split.  This is the split of K whose partial results are
 * summed on chip in the TileScale README's GEMM example (section "Example
 * of GEMM"), taken across workgroups: each workgroup accumulates its K
 * range in fp32, stores the fp32 partial tile in the workspace, and the
 * last one to finish adds the partial tiles in split order (a fixed order:
 * repeated calls give bit-identical results) and stores C.
 *   scale_a, scale_b : used for TG_IN_FP8 only (finite), ignored otherwise.
 *   workspace        : caller-owned DEVICE memory of workspace_bytes bytes,
 *                      256-byte aligned, or NULL (workspace_bytes 0: no
 *                      split, exactly the plain entry point).  Its first
 *                      64 KiB hold arrival counters: they must be zero
 *                      before the workspace's first use (zero-fill it once)
 *                      and every call leaves them zero when it completes,
 *                      so one workspace serves any later call of any shape.
 *                      The rest holds partial tiles (scratch, never cleared).
 *                      Calls that run at the same time (e.g. on two streams)
 *                      must use different workspaces.
 * Errors: TG_ERR_INVALID_VALUE for an invalid `in`, a negative
 * workspace_bytes, a NULL workspace with workspace_bytes != 0, or a
 * workspace smaller than tg_gemm_ex_workspace_bytes reports; TG_ERR_MISALIGNED
 * for a workspace not 256-byte aligned; otherwise as the plain entry point. */
tg_status tg_gemm_ex(tg_input in, int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda,
                     const void *B, int64_t ldb, tg_layout b_layout,
                     float scale_a, float scale_b,
                     void *C, int64_t ldc, tg_dtype c_dtype,
                     void *workspace, int64_t workspace_bytes,
                     void *stream);

/* tg_gemm_ex without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  It allocates nothing: its split
 * workspace is a static device array of this library, 64 MiB + 64 KiB
 * (every split plan the library makes fits in it), which each GPU holds from
 * the library's load until the process ends.  The first call with a device
 * current looks up that device's array and clears its 64 KiB of arrival
 * counters with a kernel on `stream`; every call leaves them zero.  Same
 * arguments (less the workspace), validation, results and errors as
 * tg_gemm_ex with a workspace of that size, plus TG_ERR_SCRATCH if a problem
 * would need more scratch than the array holds.  All calls on one GPU share
 * the array: calls that overlap in time on one GPU (e.g. on two streams)
 * race and must be serialized by the caller. */
tg_status tg_gemm_ex_noalloc(tg_input in, int64_t M, int64_t N, int64_t K,
                             const void *A, int64_t lda,
                             const void *B, int64_t ldb, tg_layout b_layout,
                             float scale_a, float scale_b,
                             void *C, int64_t ldc, tg_dtype c_dtype,
                             void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *tg_status_string(tg_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t tg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TG_H */
