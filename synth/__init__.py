"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no GEMM or dequant arithmetic: it only draws random numbers
with torch's CPU generator, rounds them to the storage type the workload names
(round-to-nearest-even, torch's own casts), and lays them out.  Both the HIP
path and the CPU oracle consume the same host bytes.

Workloads (sizes and distributions of the LLM GEMM / Dequant-GEMM shapes the
measured kernels are meant for; the pages print no shapes, so these stand in):

  f16_256       fp16 256^3, A and B row-major, U(-1,1), fp32 out
  bf16_4096     bf16 4096^3, A row-major, B column-major, N(0,1), bf16 out
  bf16_skinny   bf16 M=16, N=K=8192, A N(0,1), B N(0,0.02) column-major, fp32 out
  fp8_8192      e4m3 8192^3 from N(0,1), per-tensor scale amax/448, bf16 out
  w4a16         fp16 A 256x8192 N(0,1); int4 weights U{0..15} packed 8 per int32
                along K ([N][K/8]); fp16 scales U(0.005,0.02) per 128 K per
                column ([N][K/128]); zero point 8; fp16 out
  sp24_4096     bf16 M=N=K=4096, A N(0,1) row-major; 2:4 sparse weights N x K:
                kept values N(0,1) rounded to bf16 ([N][K/2]), each group's
                pair of kept positions uniform over the 6 pairs, stored as
                4-bit codes i0 | i1<<2, two per byte, low nibble first
                ([N][K/8]); bf16 out
"""
from __future__ import annotations

import torch

E4M3_MAX = 448.0

# workload name -> (seeds, description)
SEEDS = {
    "f16_256": (1, 2),
    "bf16_4096": (3, 4),
    "bf16_skinny": (5, 6),
    "fp8_8192": (7, 8),
    "w4a16": (9, 10, 11),
    "sp24_4096": (12, 13, 14),
}

# the 6 position pairs (i0 < i1) of a group of 4, as the 4-bit code i0 | i1 << 2
SP24_CODES = (0x4, 0x8, 0xC, 0x9, 0xD, 0xE)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def uniform(shape, seed: int, lo: float = -1.0, hi: float = 1.0) -> torch.Tensor:
    """float32 i.i.d. U(lo, hi)."""
    t = torch.empty(shape, dtype=torch.float32)
    t.uniform_(lo, hi, generator=_gen(seed))
    return t


def normal(shape, seed: int, std: float = 1.0) -> torch.Tensor:
    """float32 i.i.d. N(0, std^2)."""
    t = torch.empty(shape, dtype=torch.float32)
    t.normal_(0.0, std, generator=_gen(seed))
    return t


def random_words(shape, seed: int) -> torch.Tensor:
    """int32 words with uniformly random bits: every nibble is i.i.d. U{0..15}."""
    t = torch.randint(0, 1 << 16, tuple(shape) + (2,), dtype=torch.int32, generator=_gen(seed))
    return (t[..., 0] | (t[..., 1] << 16)).contiguous()


def sparse24_codes(shape, seed: int) -> torch.Tensor:
    """uint8 [rows][K/8] of 2:4 group codes: each group's pair of kept positions
    uniform over the 6 pairs, two 4-bit codes per byte, low nibble first."""
    rows, nbytes = shape
    pick = torch.randint(0, 6, (rows, nbytes, 2), generator=_gen(seed))
    codes = torch.tensor(SP24_CODES, dtype=torch.int32)[pick]
    return (codes[..., 0] | (codes[..., 1] << 4)).to(torch.uint8).contiguous()


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor e4m3 quantisation: scale = amax/448 (fp32), q = e4m3_RNE(clamp(x/scale)).

    The clamp comes first because torch's cast turns magnitudes past the
    largest finite e4m3 (448) plus half a step into NaN.
    """
    amax = x.abs().max().to(torch.float32)
    scale = (amax / E4M3_MAX).to(torch.float32)
    if float(scale) == 0.0:
        scale = torch.tensor(1.0, dtype=torch.float32)
    q = (x / scale).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q, float(scale)


def workload(name: str, M: int | None = None, N: int | None = None, K: int | None = None) -> dict:
    """Host inputs of a named workload; M, N, K override its sizes (same recipe).

    Returns a dict with 'A', 'B' (or 'qweight'/'scales'), 'M','N','K',
    'b_layout' ('row' = K x N, 'col' = N x K), 'out' ('f32','bf16','f16'),
    and for fp8 'scale_a', 'scale_b'.
    """
    if name == "f16_256":
        M, N, K = M or 256, N or 256, K or 256
        sa, sb = SEEDS[name]
        A = uniform((M, K), sa).to(torch.float16)
        B = uniform((K, N), sb).to(torch.float16)
        return dict(name=name, A=A, B=B, M=M, N=N, K=K, b_layout="row", out="f32", dtype="f16")
    if name == "bf16_4096":
        M, N, K = M or 4096, N or 4096, K or 4096
        sa, sb = SEEDS[name]
        A = normal((M, K), sa).to(torch.bfloat16)
        B = normal((N, K), sb).to(torch.bfloat16)  # column-major K x N == row-major N x K
        return dict(name=name, A=A, B=B, M=M, N=N, K=K, b_layout="col", out="bf16", dtype="bf16")
    if name == "bf16_skinny":
        M, N, K = M or 16, N or 8192, K or 8192
        sa, sb = SEEDS[name]
        A = normal((M, K), sa).to(torch.bfloat16)
        B = normal((N, K), sb, std=0.02).to(torch.bfloat16)
        return dict(name=name, A=A, B=B, M=M, N=N, K=K, b_layout="col", out="f32", dtype="bf16")
    if name == "fp8_8192":
        M, N, K = M or 8192, N or 8192, K or 8192
        sa, sb = SEEDS[name]
        Aq, scale_a = quantize_e4m3(normal((M, K), sa))
        Bq, scale_b = quantize_e4m3(normal((N, K), sb))
        return dict(name=name, A=Aq, B=Bq, M=M, N=N, K=K, b_layout="col", out="bf16",
                    dtype="fp8", scale_a=scale_a, scale_b=scale_b)
    if name == "w4a16":
        M, N, K = M or 256, N or 8192, K or 8192
        group = 128
        sa, sq, ss = SEEDS[name]
        A = normal((M, K), sa).to(torch.float16)
        qweight = random_words((N, (K + 7) // 8), sq)
        scales = uniform((N, (K + group - 1) // group), ss, 0.005, 0.02).to(torch.float16)
        return dict(name=name, A=A, qweight=qweight, scales=scales, M=M, N=N, K=K,
                    group_size=group, zero_point=8, out="f16", dtype="w4a16")
    if name == "sp24_4096":
        M, N, K = M or 4096, N or 4096, K or 4096
        sa, sv, sm = SEEDS[name]
        A = normal((M, K), sa).to(torch.bfloat16)
        vals = normal((N, K // 2), sv).to(torch.bfloat16)
        meta = sparse24_codes((N, K // 8), sm)
        return dict(name=name, A=A, vals=vals, meta=meta, M=M, N=N, K=K, out="bf16", dtype="bf16")
    raise KeyError(name)
