"""CPU oracle for the tile GEMM, the w4a16 dequant GEMM and the 2:4 sparse GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``tile_level_gemm_02_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, binary64); this module only
builds it with gcc, loads it with ctypes and marshals numpy arrays.  The
operation it computes is the plain definition C = A.B of the GEMM skeleton in
"TileScale 与 TileLang比较" (section 核心抽象与编程模型对比), and the int4
dequant of the Dequant-GEMM target kernel named in the same page (sections
设计目标、定位与适用场景, 生态互操作、性能、局限与路线图); see ``oracle.c``
for the exact formulas and the readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F16, BF16, E4M3, F64 = 0, 1, 2, 3
B_KN, B_NK = 0, 1  # B stored K x N (row-major) or N x K (column-major)

_FMT_ITEMSIZE = {F16: 2, BF16: 2, E4M3: 1, F64: 8}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
        lib.orc_expand_sp24.argtypes = [i64, i64, vp, i64, vp, i64, vp, i64]
        lib.orc_expand_sp24.restype = ctypes.c_int
        lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_f16_to_f64.restype = dp
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f64.restype = dp
        lib.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_to_f64.restype = dp
        lib.orc_f64_to_f16_rne.argtypes = [dp]
        lib.orc_f64_to_f16_rne.restype = ctypes.c_uint16
        lib.orc_f64_to_bf16_rne.argtypes = [dp]
        lib.orc_f64_to_bf16_rne.restype = ctypes.c_uint16
        lib.orc_decode.argtypes = [ctypes.c_int, vp, vp, i64]
        lib.orc_decode.restype = None
        lib.orc_encode_f16.argtypes = [vp, vp, i64]
        lib.orc_encode_f16.restype = None
        lib.orc_encode_bf16.argtypes = [vp, vp, i64]
        lib.orc_encode_bf16.restype = None
        lib.orc_dequant_w4.argtypes = [i64, i64, vp, i64, vp, i64, i32, i32, vp, i64]
        lib.orc_dequant_w4.restype = None
        lib.orc_gemm_naive.argtypes = [ctypes.c_int, i64, i64, i64, vp, i64, vp, i64,
                                       ctypes.c_int, dp, dp, vp, vp, i64]
        lib.orc_gemm_naive.restype = None
        lib.orc_gemm.argtypes = [ctypes.c_int, i64, i64, i64, vp, i64, vp, i64,
                                 ctypes.c_int, dp, dp, vp, vp, i64, ctypes.c_int]
        lib.orc_gemm.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _bits(a, itemsize: int) -> np.ndarray:
    """Return a C-contiguous numpy view of raw element bits (uint8/uint16/float64)."""
    if hasattr(a, "numpy"):  # a torch CPU tensor
        import torch  # local: the oracle itself never needs torch

        if a.dtype in (torch.float16, torch.bfloat16):
            a = a.contiguous().view(torch.int16).numpy().view(np.uint16)
        elif a.dtype == torch.float8_e4m3fn:
            a = a.contiguous().view(torch.uint8).numpy()
        else:
            a = a.contiguous().numpy()
    a = np.ascontiguousarray(a)
    if itemsize == 2:
        return a.view(np.uint16)
    if itemsize == 1:
        return a.view(np.uint8)
    if itemsize == 4:
        return a.view(np.int32)
    return a.astype(np.float64, copy=False)


# ------------------------------------------------------------------ codecs

def decode(fmt: int, bits) -> np.ndarray:
    """Exact binary64 values of stored elements of format ``fmt``."""
    lib = _load()
    b = _bits(bits, _FMT_ITEMSIZE[fmt])
    out = np.empty(b.shape, dtype=np.float64)
    lib.orc_decode(fmt, _ptr(b), _ptr(out), b.size)
    return out


def encode_f16(x) -> np.ndarray:
    """binary64 -> IEEE binary16 bits, one round-to-nearest-even step."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.orc_encode_f16(_ptr(x), _ptr(out), x.size)
    return out


def encode_bf16(x) -> np.ndarray:
    """binary64 -> bfloat16 bits, one round-to-nearest-even step (never via fp32)."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.orc_encode_bf16(_ptr(x), _ptr(out), x.size)
    return out


# ------------------------------------------------------------------ dequant

def dequant_w4(qweight, scales, K: int, group_size: int = 128, zero_point: int = 8) -> np.ndarray:
    """fp16 bits W[N][K] of the int4 weights.

    ``qweight`` int32 [N][ceil(K/8)] (nibble j of word w is k = 8w + j),
    ``scales`` fp16 bits [N][ceil(K/group_size)].
    """
    lib = _load()
    q = _bits(qweight, 4)
    s = _bits(scales, 2)
    N = q.shape[0]
    W = np.empty((N, K), dtype=np.uint16)
    lib.orc_dequant_w4(N, K, _ptr(q), q.shape[1], _ptr(s), s.shape[1], group_size,
                       zero_point, _ptr(W), K)
    return W


# ------------------------------------------------------------------- GEMM

def gemm(fmt: int, A, B, b_layout: int, scale_a: float = 1.0, scale_b: float = 1.0,
         nthreads: int | None = None, naive: bool = False):
    """C, S (binary64, M x N) for C = scale_a*scale_b * A.B.

    ``A`` is M x K (row-major), ``B`` is K x N when ``b_layout == B_KN`` or
    N x K when ``b_layout == B_NK``; elements are stored bits of ``fmt``.
    """
    lib = _load()
    isz = _FMT_ITEMSIZE[fmt]
    a = _bits(A, isz)
    b = _bits(B, isz)
    M, K = a.shape
    if b_layout == B_KN:
        assert b.shape[0] == K
        N = b.shape[1]
    else:
        assert b.shape[1] == K
        N = b.shape[0]
    C = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    if M == 0 or N == 0:
        return C, S
    if naive:
        lib.orc_gemm_naive(fmt, M, N, K, _ptr(a), K, _ptr(b), b.shape[1], b_layout,
                           float(scale_a), float(scale_b), _ptr(C), _ptr(S), N)
        return C, S
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    rc = lib.orc_gemm(fmt, M, N, K, _ptr(a), K, _ptr(b), b.shape[1], b_layout,
                      float(scale_a), float(scale_b), _ptr(C), _ptr(S), N, int(nthreads))
    if rc != 0:
        raise MemoryError("oracle gemm: out of memory")
    return C, S


# ------------------------------------------------------- 2:4 sparse weights

def expand_sp24(vals, meta, K: int) -> np.ndarray:
    """bf16 (or fp16) bits W[N][K] of 2:4-compressed weights (format in oracle.c).

    ``vals`` 16-bit [N][K/2] (the kept values of each group of 4, in position
    order), ``meta`` uint8 [N][K/8] (a 4-bit code i0 | i1 << 2 per group, low
    nibble first).  Raises ValueError on a code with i0 >= i1.
    """
    lib = _load()
    v = _bits(vals, 2)
    m = np.ascontiguousarray(meta.numpy() if hasattr(meta, "numpy") else meta, dtype=np.uint8)
    N = v.shape[0]
    assert K % 4 == 0 and v.shape[1] >= K // 2 and m.shape[1] >= (K + 7) // 8 and m.shape[0] == N
    W = np.empty((N, K), dtype=np.uint16)
    if lib.orc_expand_sp24(N, K, _ptr(v), v.shape[1], _ptr(m), m.shape[1], _ptr(W), K) != 0:
        raise ValueError("2:4 metadata: a group code with i0 >= i1")
    return W


def compress_sp24(W_bits) -> tuple:
    """(vals, meta) of an N x K matrix of 16-bit element bits whose every group
    of 4 along K has at most 2 nonzero entries (bits other than +-0); unused
    slots take the lowest free positions.  Pure Python: small inputs only."""
    W = np.asarray(_bits(W_bits, 2))
    N, K = W.shape
    vals = np.zeros((N, K // 2), dtype=np.uint16)
    meta = np.zeros((N, (K + 7) // 8), dtype=np.uint8)
    for n in range(N):
        for g in range(K // 4):
            grp = W[n, 4 * g: 4 * g + 4]
            keep = [j for j in range(4) if grp[j] & 0x7FFF]
            if len(keep) > 2:
                raise ValueError(f"row {n} group {g}: more than 2 nonzeros")
            for j in range(4):
                if len(keep) < 2 and j not in keep:
                    keep.append(j)
            i0, i1 = sorted(keep[:2])
            vals[n, 2 * g], vals[n, 2 * g + 1] = grp[i0], grp[i1]
            meta[n, g // 2] |= (i0 | (i1 << 2)) << (4 * (g % 2))
    return vals, meta


def gemm_sp24(A, vals, meta, K: int, fmt: int = BF16, nthreads: int | None = None):
    """C, S for C = A . W^T with W the expanded 2:4 weights (N x K, K-contiguous)."""
    W = expand_sp24(vals, meta, K)
    return gemm(fmt, A, W, B_NK, nthreads=nthreads)


def w4a16(A, qweight, scales, K: int, group_size: int = 128, zero_point: int = 8,
          nthreads: int | None = None):
    """C, S for the w4a16 GEMM: dequant W (fp16 [N][K]) then the fp16 GEMM A.W^T."""
    W = dequant_w4(qweight, scales, K, group_size, zero_point)
    return gemm(F16, A, W, B_NK, nthreads=nthreads)
