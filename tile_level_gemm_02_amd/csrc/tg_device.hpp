// Device-side building blocks shared by the tile GEMM kernels (gfx950 only).
//
// The kernels follow the dataflow of the single-GPU GEMM skeleton in
// "TileScale 与 TileLang比较" (section 核心抽象与编程模型对比): one workgroup per
// output tile, A and B K-slices staged in on-chip shared memory (LDS here), a
// register accumulator cleared before the K loop, one tile product per K step,
// one store of the accumulator at the end.  The compiler passes listed in the
// section 编译与优化流水线 (shared-memory swizzle, vectorised copies,
// software pipelining, tensorisation, tail splitting) are written out by hand
// in these files for CDNA4: XOR-swizzled LDS rows, 128-bit global loads,
// double-buffered LDS, MFMA instructions, and masked tails.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef int v2i32_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// element type of A and B
enum Elem : int { E_F16 = 0, E_BF16 = 1, E_FP8 = 2 };
// output type of C
enum Out : int { O_F32 = 0, O_F16 = 1, O_BF16 = 2 };

template <int E> struct ElemInfo;
template <> struct ElemInfo<E_F16> { static constexpr int bytes = 2; };
template <> struct ElemInfo<E_BF16> { static constexpr int bytes = 2; };
template <> struct ElemInfo<E_FP8> { static constexpr int bytes = 1; };

template <typename T, typename F> __device__ __forceinline__ T bit_cast(F f)
{
    static_assert(sizeof(T) == sizeof(F), "size");
    return __builtin_bit_cast(T, f);
}

// ------------------------------------------------------------------ MFMA
// One 32x32 output block += (32 x kstep) . (kstep x 32).  Lane l holds row
// (l % 32) of A and column (l % 32) of B; both operands carry the same k
// values per lane and register, so the k order inside a step is irrelevant
// to the sum.  16-bit types: kstep 16, 8 elements per lane.  fp8: kstep 64,
// 32 elements per lane.
template <int E> struct Mfma32;
template <> struct Mfma32<E_F16> {
    typedef u32x4 frag;
    __device__ __forceinline__ static f32x16 run(frag a, frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(bit_cast<f16x8>(a), bit_cast<f16x8>(b), c, 0, 0, 0);
    }
};
template <> struct Mfma32<E_BF16> {
    typedef u32x4 frag;
    __device__ __forceinline__ static f32x16 run(frag a, frag b, f32x16 c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bit_cast<bf16x8>(a), bit_cast<bf16x8>(b), c, 0, 0, 0);
    }
};
template <> struct Mfma32<E_FP8> {
    typedef i32x8 frag;
    __device__ __forceinline__ static f32x16 run(frag a, frag b, f32x16 c)
    {
        // format codes 0/0: both operands OCP e4m3; scale arguments unused (0)
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

// Wait states between the last MFMA of a kernel and the first instruction that
// reads its accumulators.  A 16-pass MFMA (the fp8 32x32x64 form) needs 18
// before a VALU, VMEM or LDS instruction may read its result; 24 are spent
// here unconditionally, once per kernel, instead of relying on the count the
// compiler derives (a short count was observed for the fp8 form).
__device__ __forceinline__ void mfma_drain()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------- output conversion
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x)
{
    uint32_t u = bit_cast<uint32_t>(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0;  // NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float x)
{
    return bit_cast<uint16_t>((_Float16)x);
}

template <int O> struct OutInfo;
template <> struct OutInfo<O_F32> { typedef float T; };
template <> struct OutInfo<O_F16> { typedef uint16_t T; };
template <> struct OutInfo<O_BF16> { typedef uint16_t T; };

template <int O> __device__ __forceinline__ typename OutInfo<O>::T convert_out(float x);
template <> __device__ __forceinline__ float convert_out<O_F32>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t convert_out<O_F16>(float x) { return f32_to_f16_rne(x); }
template <> __device__ __forceinline__ uint16_t convert_out<O_BF16>(float x) { return f32_to_bf16_rne(x); }

// ------------------------------------------------------------ LDS swizzle
// A staged tile row holds 128 bytes of K (8 chunks of 16 bytes).  Chunk c of
// row r lives at chunk position c ^ (r & 7), so the 8 lanes that read one
// chunk column from 8 consecutive rows hit 8 different 16-byte bank groups.
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk)
{
    return row * 128u + ((chunk ^ (row & 7u)) << 4);
}

// -------------------------------------------------------- masked loading
// Load the 16-byte chunk of a K-contiguous row that starts at element k0,
// keeping only elements with index < kmax (bytes beyond are zero).  Used
// only on tails, where the full 16 bytes may run past the buffer.
template <int EB>
__device__ __forceinline__ u32x4 load_chunk_partial(const uint8_t* p, int64_t avail)
{
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 16 / EB; ++e) {
        if (e < avail) {
            uint32_t v = (EB == 2) ? (uint32_t)((const uint16_t*)p)[e] : (uint32_t)p[e];
            w[(e * EB) >> 2] |= v << (((e * EB) & 3) * 8);
        }
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ u32x4 ldg128(const void* p)
{
    return *(const u32x4*)p;
}

__device__ __forceinline__ void sts128(uint8_t* lds, uint32_t off, u32x4 v)
{
    *(u32x4*)(lds + off) = v;
}

__device__ __forceinline__ u32x4 lds128(const uint8_t* lds, uint32_t off)
{
    return *(const u32x4*)(lds + off);
}

// Store of output data that this kernel never reads back, marked non-temporal
// (streaming): measured ~1% faster than a plain store for the 32 MB bf16
// output of the 4096^3 GEMM.
template <typename T>
__device__ __forceinline__ void store_nt(T* p, T v)
{
    __builtin_nontemporal_store(v, p);
}

// ------------------------------------------------------------ int4 dequant
// Eight int4 weights of one 32-bit word -> eight fp16 values, in k order
// (nibble j, bits 4j..4j+3, is k offset j), W = fp16_RNE((q - zp) * s).
// Per byte (two nibbles, k offsets 2j and 2j+1):
//   t = [byte j, 0, byte j, 0]                      (one byte permute)
//   x = (t & 0x00F0000F) | 0x64006400               (one and-or)
//     low half  = fp16 1024 + q_lo    (q in the fraction's low bits)
//     high half = fp16 1024 + 16*q_hi (q four bits up)
//   h = x * (1, 1/16) + (-(1024+zp), -(64+zp))      (packed fma: exact, the
//     result q - zp is a small integer)
//   w = h * (s, s)                                  (packed multiply: the one
//     round-to-nearest-even step)
struct W4Consts {
    f16x2 mul;      // (1, 1/16)
    f16x2 bias;     // (-(1024 + zp), -(64 + zp))
    uint32_t mask;  // 0x00F0000F, held in a vector register
};

__device__ __forceinline__ W4Consts w4_consts(int zero_point)
{
    W4Consts c;
    c.mul = f16x2{(_Float16)1.0f, (_Float16)0.0625f};
    c.bias = f16x2{(_Float16)(-(1024 + zero_point)), (_Float16)(-(64 + zero_point))};  // exact
    // in a register, so the and-or below is one instruction (its three-operand
    // form takes no literal and at most one scalar operand)
    asm("v_mov_b32 %0, 0x00F0000F" : "=v"(c.mask));
    return c;
}

__device__ __forceinline__ u32x4 dequant_w4_word(uint32_t w, W4Consts c, f16x2 s2)
{
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t sel = 0x0C000C00u | ((uint32_t)j << 16) | (uint32_t)j;
        const uint32_t t = __builtin_amdgcn_perm(0u, w, sel);
        uint32_t x;  // (t & 0x00F0000F) | 0x64006400
        asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(x) : "v"(t), "v"(c.mask), "s"(0x64006400u));
        const f16x2 h = __builtin_elementwise_fma(bit_cast<f16x2>(x), c.mul, c.bias);
        out[j] = bit_cast<uint32_t>(h * s2);
    }
    return u32x4{out[0], out[1], out[2], out[3]};
}

// ------------------------------------------------------- tile scheduling
// Workgroups are dealt to the 8 XCDs of the chip round-robin (id % 8).
// Consecutive ids are regrouped so that each XCD receives a contiguous range
// of the work (when the grid is a multiple of 8).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nblocks)
{
    return (nblocks & 7u) == 0u ? (bid & 7u) * (nblocks >> 3) + (bid >> 3) : bid;
}

// Tile r (0 .. tiles_m*tiles_n - 1) of a walk that takes group_m tile rows
// at a time, so that tiles resident together share rows of A and columns
// of B in their XCD's L2.
__device__ __forceinline__ void group_walk(uint32_t r, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m,
                                           uint32_t& tm, uint32_t& tn)
{
    uint32_t per_group = group_m * tiles_n;
    uint32_t g = r / per_group;
    uint32_t first_m = g * group_m;
    uint32_t gsize = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    uint32_t q = r - g * per_group;
    tm = first_m + q % gsize;
    tn = q / gsize;
}

// Map the linear workgroup id to an output tile (XCD-aware, grouped walk).
__device__ __forceinline__ void tile_coords(uint32_t bid, uint32_t nblocks, uint32_t tiles_m,
                                            uint32_t tiles_n, uint32_t group_m, uint32_t& tm,
                                            uint32_t& tn)
{
    group_walk(xcd_remap(bid, nblocks), tiles_m, tiles_n, group_m, tm, tn);
}

// With K split over `splits` workgroups per tile (the grid is tiles x
// splits): the remapped id gives the split (slowest) and the tile, so an
// XCD's contiguous range holds neighbouring tiles of one K range, which
// share their A and B K-slices in its L2.
__device__ __forceinline__ void tile_split_coords(uint32_t bid, uint32_t nblocks, uint32_t tiles_m,
                                                  uint32_t tiles_n, uint32_t splits, uint32_t group_m,
                                                  uint32_t& tm, uint32_t& tn, uint32_t& split)
{
    const uint32_t idx = xcd_remap(bid, nblocks), tiles = tiles_m * tiles_n;
    split = idx / tiles;
    group_walk(idx - split * tiles, tiles_m, tiles_n, group_m, tm, tn);
    (void)splits;
}

// ------------------------------------------------------ split-K handoff
// A K range split over S workgroups per output tile (the TileScale
// README's split of K whose partial results are summed on chip, section
// "Example of GEMM", taken across workgroups): each wave that owns a share
// of the tile stores its fp32 partial share in a workspace slot of its own,
// then counts itself in at the share's arrival counter.  The wave that
// arrives last adds the S partials in split order (a fixed order: the
// result does not depend on which wave arrives last), resets the counter to
// zero for the next call, and stores the share.  No wave ever waits for
// another.
//
// Layout of a partial share in its slot: value v = 4g + e of accumulator
// block b of lane l at float ((b*4 + g)*64 + l)*4 + e, so each wave store
// and load moves 1 KiB of contiguous memory.
//
// Coherence across the chip's 8 XCDs (each with its own L2): the partial
// shares are stored and loaded with the device-scope cache policy (sc1), the
// bits the compiler gives relaxed agent-scope atomic stores and loads:
// stores write through to the device-coherent level, loads do not hit a
// stale L2 line.  So publishing needs only the completion of this wave's
// stores before it counts in, and the last arrival's loads see every
// partial once its count says all have arrived -- no whole-L2 write-back or
// invalidate (buffer_wbl2 / buffer_inv), which made a split launch slower
// than none.
constexpr int kCachePolicyDevice = 16;  // sc1

__device__ __forceinline__ void splitk_store(float* slot, int b, int g, uint32_t lane, f32x4 v)
{
    const auto r = __builtin_amdgcn_make_buffer_rsrc((void*)slot, (short)0, 0x7FFFFFF0, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(bit_cast<u32x4>(v), r, (int)(((b * 4 + g) * 64 + lane) * 16), 0,
                                           kCachePolicyDevice);
}

__device__ __forceinline__ f32x4 splitk_load(const float* slot, int b, int g, uint32_t lane)
{
    const auto r = __builtin_amdgcn_make_buffer_rsrc((void*)slot, (short)0, 0x7FFFFFF0, 0x00020000);
    return bit_cast<f32x4>(
        __builtin_amdgcn_raw_buffer_load_b128(r, (int)(((b * 4 + g) * 64 + lane) * 16), 0, kCachePolicyDevice));
}

// Called by every lane of a wave after it stored its partial share; true
// (in every lane) for the last of the `splits` arrivals at `counter`.  The
// wave's partial stores have completed (vmcnt 0) before it counts itself in
// with a device-scope atomic; the last arrival's loads come after its count.
__device__ __forceinline__ bool splitk_last(uint32_t* counter, uint32_t splits, uint32_t lane)
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    uint32_t old = 0u;
    if (lane == 0u)
        old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readlane(old, 0);
    asm volatile("" ::: "memory");  // no load of a partial is moved above the count
    if (old != splits - 1u)
        return false;
    // every partial of this share has arrived: the counter is free again
    if (lane == 0u)
        __hip_atomic_exchange(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

}  // namespace tg
