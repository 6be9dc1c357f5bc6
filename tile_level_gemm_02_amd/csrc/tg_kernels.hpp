// Kernel templates of the tile GEMM library (gfx950).
//
//  tile_gemm   : the tiled MFMA GEMM for fp16 / bf16 / fp8 and, with W4, the
//                w4a16 Dequant-GEMM.  Dataflow of the single-GPU GEMM
//                skeleton in "TileScale 与 TileLang比较" (section
//                核心抽象与编程模型对比): grid of output tiles, global->LDS copy
//                of one K slice of A and of B per step, tile product into a
//                cleared register accumulator, pipelined K loop, one store.
//  dequant_w4  : the int4 -> fp16 dequant step alone, using the very routine
//                the w4a16 GEMM uses.
#pragma once

#include "tg_device.hpp"

namespace tg {

struct TileArgs {
    int64_t M, N, K;
    const uint8_t* A;
    int64_t lda;  // elements
    const uint8_t* B;
    int64_t ldb;  // elements
    void* C;
    int64_t ldc;  // elements
    float alpha;  // fp8 only: scale_a * scale_b
    uint32_t group_m;
    // w4a16 only
    const uint32_t* qw;
    int64_t ldq;  // int32 words
    const uint16_t* scales;
    int64_t lds;  // fp16 elements
    int32_t zero_point;
    // K split over `splits` workgroups per output tile (1: no split).  With
    // splits > 1 the kernel takes one arrival counter per tile and wave from
    // `counters` (all zero on entry, zero again on exit) and one fp32 partial
    // share per tile, split and wave from `partials` (see splitk_last).
    uint32_t splits;
    uint32_t* counters;
    float* partials;
    // NT kernel only: with dp > 0 the first dp workgroups run the first dp
    // tiles of the walk whole, and only the remaining tiles split K `splits`
    // ways (counters and partial shares are then numbered from tile dp).
    uint32_t dp;
    // NT kernel with tiles smaller than 256 x 256 only: with sub256 > 0,
    // the Q = (256 / BM) x (256 / BN) parts of each 256 x 256 tile of the
    // 256 x 256 walk from position sub256 - 1 on (the tiles that a 256 x 256
    // launch of the first sub256 - 1 tiles left over): workgroup j takes
    // part j % Q (row-major) of tile sub256 - 1 + j / Q.
    uint32_t sub256;
};

// B storage: K-contiguous (column-major K x N, i.e. N x K rows) or N-contiguous
enum BLay : int { B_KCONTIG = 0, B_NCONTIG = 1 };

constexpr int kThreads = 256;  // 4 waves, arranged 2 x 2 over the output tile

// --------------------------------------------------------------------------
// Tiled GEMM.  One workgroup computes a BM x BN tile of C.  Each K step
// stages 128 bytes of K per row (64 fp16/bf16 or 128 fp8 elements) of the A
// tile (BM rows) and the B tile (BN columns, stored K-contiguous in LDS) in a
// double-buffered, XOR-swizzled LDS ring.  While the MFMAs consume one
// buffer, the 128-bit global loads of the next K step are in flight in
// registers; they are written to the other buffer after the MFMAs, then one
// barrier flips the buffers.
// --------------------------------------------------------------------------
template <int E, int BL, int O, int BM, int BN, bool W4>
__global__ __launch_bounds__(kThreads) void tile_gemm(TileArgs p)
{
    constexpr int EB = ElemInfo<E>::bytes;
    constexpr int CE = 16 / EB;   // elements per 16-byte chunk
    constexpr int KE = 128 / EB;  // K elements per step
    constexpr int TM = BM / 64;   // 32x32 blocks per wave along M
    constexpr int TN = BN / 64;   // and along N
    constexpr int A_CH = BM * 8 / kThreads;
    constexpr int B_CH = BN * 8 / kThreads;
    constexpr int KSTEPS = (E == E_FP8) ? 2 : 4;  // MFMAs along K per step
    static_assert(!W4 || (E == E_F16 && BL == B_KCONTIG), "w4a16 uses fp16 A and K-packed weights");
    static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");
    typedef typename Mfma32<E>::frag Frag;
    typedef typename OutInfo<O>::T OutT;

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * 128];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const int64_t M = p.M, N = p.N, K = p.K;
    const uint32_t tiles_m = (uint32_t)((M + BM - 1) / BM);
    const uint32_t tiles_n = (uint32_t)((N + BN - 1) / BN);
    uint32_t tmi, tni;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, p.group_m, tmi, tni);
    const int64_t m0 = (int64_t)tmi * BM;
    const int64_t n0 = (int64_t)tni * BN;
    const int64_t KT = (K + KE - 1) / KE;

    u32x4 ra[A_CH];
    u32x4 rb[W4 ? 1 : B_CH];
    uint32_t rq[W4 ? B_CH : 1];
    uint16_t rs[W4 ? B_CH : 1];

    // ---- global -> registers, one K step
    auto load_a = [&](int64_t kt) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const uint32_t idx = tid + kThreads * i;
            const int64_t gm = m0 + (idx >> 3);
            const int64_t gk = kt * KE + (int64_t)(idx & 7u) * CE;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (gm < M && gk < K) {
                const uint8_t* src = p.A + (gm * p.lda + gk) * EB;
                v = (gk + CE <= K) ? ldg128(src) : load_chunk_partial<EB>(src, K - gk);
            }
            ra[i] = v;
        }
    };
    auto load_b = [&](int64_t kt) {
        if constexpr (W4) {
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const uint32_t idx = tid + kThreads * i;
                const int64_t gn = n0 + (idx >> 3);
                uint32_t q = 0u;
                uint16_t s = 0;
                if (gn < N) {  // K is a multiple of 128: every step is full
                    q = p.qw[gn * p.ldq + kt * 8 + (idx & 7u)];
                    s = p.scales[gn * p.lds + ((kt * KE) >> 7)];
                }
                rq[i] = q;
                rs[i] = s;
            }
        } else if constexpr (BL == B_KCONTIG) {
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const uint32_t idx = tid + kThreads * i;
                const int64_t gn = n0 + (idx >> 3);
                const int64_t gk = kt * KE + (int64_t)(idx & 7u) * CE;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (gn < N && gk < K) {
                    const uint8_t* src = p.B + (gn * p.ldb + gk) * EB;
                    v = (gk + CE <= K) ? ldg128(src) : load_chunk_partial<EB>(src, K - gk);
                }
                rb[i] = v;
            }
        } else {
            constexpr int NCH = BN / CE;  // chunks along one B row (fixed k)
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const uint32_t idx = tid + kThreads * i;
                const int64_t gk = kt * KE + idx / NCH;
                const int64_t gn = n0 + (int64_t)(idx % NCH) * CE;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (gk < K && gn < N) {
                    const uint8_t* src = p.B + (gk * p.ldb + gn) * EB;
                    v = (gn + CE <= N) ? ldg128(src) : load_chunk_partial<EB>(src, N - gn);
                }
                rb[i] = v;
            }
        }
    };
    // ---- registers -> LDS buffer `buf`
    auto store_ab = [&](int buf) {
        uint8_t* As = smem + buf * (BM + BN) * 128;
        uint8_t* Bs = As + BM * 128;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const uint32_t idx = tid + kThreads * i;
            sts128(As, swz(idx >> 3, idx & 7u), ra[i]);
        }
        if constexpr (W4) {
            const W4Consts wc = w4_consts(p.zero_point);
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const uint32_t idx = tid + kThreads * i;
                const _Float16 s = bit_cast<_Float16>(rs[i]);
                sts128(Bs, swz(idx >> 3, idx & 7u), dequant_w4_word(rq[i], wc, f16x2{s, s}));
            }
        } else if constexpr (BL == B_KCONTIG) {
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const uint32_t idx = tid + kThreads * i;
                sts128(Bs, swz(idx >> 3, idx & 7u), rb[i]);
            }
        } else {
            // transpose on the way in: element (k, n) goes to LDS row n at byte k*EB
            constexpr int NCH = BN / CE;
#pragma unroll
            for (int i = 0; i < B_CH; ++i) {
                const uint32_t idx = tid + kThreads * i;
                const uint32_t kr = idx / NCH;
                const uint32_t nb = (idx % NCH) * CE;
                const uint32_t kbyte = kr * EB;
#pragma unroll
                for (int e = 0; e < CE; ++e) {
                    const uint32_t word = rb[i][(e * EB) >> 2];
                    const uint32_t v = word >> (((e * EB) & 3) * 8);
                    const uint32_t off = swz(nb + e, kbyte >> 4) + (kbyte & 15u);
                    if constexpr (EB == 2)
                        *(uint16_t*)(Bs + off) = (uint16_t)v;
                    else
                        *(uint8_t*)(Bs + off) = (uint8_t)v;
                }
            }
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = f32x16{};

    const uint32_t wm = wave >> 1, wn = wave & 1u;
    const uint32_t rowA0 = wm * (BM / 2), rowB0 = wn * (BN / 2);
    const uint32_t lrow = lane & 31u, lgrp = lane >> 5;

    // ---- one K step of MFMAs out of LDS buffer `buf`
    auto compute = [&](int buf) {
        const uint8_t* As = smem + buf * (BM + BN) * 128;
        const uint8_t* Bs = As + BM * 128;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            Frag a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const uint32_t row = rowA0 + i * 32 + lrow;
                if constexpr (E == E_FP8) {
                    const u32x4 lo = lds128(As, swz(row, 4 * s + 2 * lgrp));
                    const u32x4 hi = lds128(As, swz(row, 4 * s + 2 * lgrp + 1));
                    a[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                } else {
                    a[i] = lds128(As, swz(row, 2 * s + lgrp));
                }
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const uint32_t row = rowB0 + j * 32 + lrow;
                if constexpr (E == E_FP8) {
                    const u32x4 lo = lds128(Bs, swz(row, 4 * s + 2 * lgrp));
                    const u32x4 hi = lds128(Bs, swz(row, 4 * s + 2 * lgrp + 1));
                    b[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                } else {
                    b[j] = lds128(Bs, swz(row, 2 * s + lgrp));
                }
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = Mfma32<E>::run(a[i], b[j], acc[i][j]);
        }
    };

    if (KT > 0) {
        load_a(0);
        load_b(0);
        store_ab(0);
    }
    __syncthreads();
    for (int64_t kt = 0; kt < KT; ++kt) {
        const int cur = (int)(kt & 1);
        const bool more = kt + 1 < KT;
        if (more) {
            load_a(kt + 1);
            load_b(kt + 1);
        }
        compute(cur);
        if (more)
            store_ab(cur ^ 1);
        __syncthreads();
    }

    mfma_drain();

    // ---- epilogue: accumulator block (32x32, 16 values per lane) -> C
    // value v of lane l sits at row 8*(v/4) + 4*(l/32) + v%4, column l%32
    OutT* C = (OutT*)p.C;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + rowB0 + j * 32 + lrow;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + rowA0 + i * 32 + (v >> 2) * 8 + lgrp * 4 + (v & 3);
                float x = acc[i][j][v];
                if constexpr (E == E_FP8)
                    x *= p.alpha;
                if (row < M && col < N)
                    C[row * p.ldc + col] = convert_out<O>(x);
            }
        }
    }
}

// --------------------------------------------------------------------------
// Arguments of the skinny GEMM (M <= 16 against a K-contiguous B; the kernel
// is in tg_gemm_skinny.hpp), and the 16x16x32 matrix instruction it and the
// w4a16 decode kernels use.
// --------------------------------------------------------------------------
struct SkinnyArgs {
    int64_t M, N, K;
    const uint8_t* A;
    int64_t lda;
    const uint8_t* B;
    int64_t ldb;
    void* C;
    int64_t ldc;
    // K split through a workspace (see skinny_gemm, SPLIT = 2): one arrival
    // counter per workgroup column, one 1 KiB partial tile per workgroup
    uint32_t* counters;
    float* partials;
};

template <int E> struct Mfma16;
template <> struct Mfma16<E_F16> {
    __device__ __forceinline__ static f32x4 run(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(bit_cast<f16x8>(a), bit_cast<f16x8>(b), c, 0, 0, 0);
    }
};
template <> struct Mfma16<E_BF16> {
    __device__ __forceinline__ static f32x4 run(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bit_cast<bf16x8>(a), bit_cast<bf16x8>(b), c, 0, 0, 0);
    }
};

// Zero an M x N fp32 matrix with leading dimension ldc (the split skinny
// GEMM adds its partial tiles into it); rows start 16-byte aligned.  Grid:
// ceil(N / 1024) x M workgroups, 4 columns per lane.  A template only so
// that every translation unit that launches it may define it.
template <int = 0>
__global__ __launch_bounds__(256) void zero_f32(float* C, int64_t N, int64_t ldc)
{
    const int64_t col = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    float* row = C + (int64_t)blockIdx.y * ldc;
    if (col + 4 <= N) {
        *(f32x4*)(row + col) = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
        for (int64_t c = col; c < N; ++c)
            row[c] = 0.0f;
    }
}

// --------------------------------------------------------------------------
// Dequant alone: one thread per 32-bit word of qweight -> 8 fp16 of W[n][k].
// --------------------------------------------------------------------------
struct DequantArgs {
    int64_t N, K;
    const uint32_t* qw;
    int64_t ldq;
    const uint16_t* scales;
    int64_t lds;
    int32_t group_size, zero_point;
    uint16_t* W;
    int64_t ldw;
};

__global__ void dequant_w4_kernel(DequantArgs p);  // defined in tg_w4a16.hip

}  // namespace tg
