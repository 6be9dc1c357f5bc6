"""tg_gemm_ex_noalloc (the split GEMM with the library's static scratch in
place of a caller workspace) against tg_gemm_ex with a caller workspace,
through the C ABI: calls in a row, each smaller than the one before, on
split plans of both kernels that split (the NT tile kernel and the skinny
kernel) and on one that does not.  Each output must equal tg_gemm_ex's bit
for bit (same plan, same kernels, same split order) and meet the oracle's
bound."""
import pytest
import torch

import oracle
import synth
from oracle import check as ochk

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "f16": torch.float16}
FMT = {"bf16": oracle.BF16, "fp8": oracle.E4M3, "f16": oracle.F16}


@pytest.fixture(scope="module")
def tg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_gemm_02_amd as tg

    return tg


def _inputs(dt, M, N, K, seed):
    if dt == "fp8":
        A, sa = synth.quantize_e4m3(synth.normal((M, K), seed))
        B, sb = synth.quantize_e4m3(synth.normal((N, K), seed + 1))
        return A, B, sa, sb
    return synth.normal((M, K), seed).to(TDT[dt]), synth.normal((N, K), seed + 1, std=0.05).to(TDT[dt]), 1.0, 1.0


def _pair(tg, dt, out, M, N, K, seed):
    """(noalloc output, tg_gemm_ex output, inputs) for one problem."""
    A, B, sa, sb = _inputs(dt, M, N, K, seed)
    dA, dB = A.cuda(), B.cuda()
    odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out]
    C1 = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    tg.tg_gemm_ex_noalloc(dA, dB, C1, b_layout="col", scale_a=sa, scale_b=sb)
    need = tg.tg_gemm_ex_workspace_bytes(TDT[dt], M, N, K)
    ws = torch.zeros(max(need, 256) // 4, dtype=torch.int32, device="cuda")
    C2 = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    tg.tg_gemm_ex(dA, dB, C2, b_layout="col", scale_a=sa, scale_b=sb, workspace=ws)
    torch.cuda.synchronize()
    return C1, C2, (A, B, sa, sb), need


# in a row, each smaller than the one before: a last round of 68 tiles of
# 256 x 256 split 3 ways behind 256 whole tiles (51 MiB of scratch), a split
# of every tile (16 MiB of partial tiles), a smaller one on the 64 tile, an
# fp8 one, the skinny kernel's split with a 16-bit output (16 columns per
# workgroup, then 32 in two row slices), and a problem that does not split
CALLS = [("bf16", "bf16", 4400, 4504, 4104), ("bf16", "bf16", 256, 8192, 8192), ("bf16", "bf16", 64, 1024, 8192),
         ("fp8", "f32", 40, 1000, 4096),
         ("bf16", "bf16", 16, 1024, 8192), ("f16", "f16", 24, 520, 4096), ("f16", "f16", 9, 200, 1000)]


def test_noalloc_matches_gemm_ex_in_a_row(tg):
    for i, (dt, out, M, N, K) in enumerate(CALLS):
        print(f"noalloc call {i}: {dt} {M}x{N}x{K} -> {out}", flush=True)
        C1, C2, (A, B, sa, sb), need = _pair(tg, dt, out, M, N, K, seed=100 + i)
        if i < len(CALLS) - 1:
            assert need > 0, "expected a split plan"
        eq = torch.equal(C1.view(torch.int16), C2.view(torch.int16)) if out != "f32" else torch.equal(C1, C2)
        assert eq, f"call {i}: noalloc output differs from tg_gemm_ex"
        cref, S = oracle.gemm(FMT[dt], A, B, oracle.B_NK, sa, sb)
        ok, r, idx = ochk.check(C1.float().cpu().double().numpy(), cref, S, K, out)
        assert ok, (i, r, idx)


def test_noalloc_repeats_bitwise(tg):
    """The scratch keeps the last call's partials and its counters return to
    zero: a repeat of the largest split plan after smaller ones is bit-identical."""
    C1, _, _, _ = _pair(tg, "bf16", "bf16", 256, 8192, 8192, seed=100)
    C3, _, _, _ = _pair(tg, "bf16", "bf16", 256, 8192, 8192, seed=100)
    assert torch.equal(C1.view(torch.int16), C3.view(torch.int16))


def test_noalloc_under_graph_capture(tg):
    """The use the entry point is for: a call captured in a HIP graph (nothing
    allocated inside the capture) and replayed, with eager work and
    synchronizations between the replays; each replay, on new contents of A,
    equals an eager call on the same inputs bit for bit."""
    M, N, K = 256, 8192, 8192
    _, B, _, _ = _inputs("bf16", M, N, K, seed=300)
    dB = B.cuda()
    dA = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    Ce = torch.empty_like(C)
    dA.copy_(synth.normal((M, K), 301).to(torch.bfloat16))
    tg.tg_gemm_ex_noalloc(dA, dB, Ce, b_layout="col")  # eager first call: the scratch is set up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tg.tg_gemm_ex_noalloc(dA, dB, C, b_layout="col")
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"graph replay {rep}", flush=True)
        dA.copy_(synth.normal((M, K), 302 + rep).to(torch.bfloat16))
        tg.tg_gemm_ex_noalloc(dA, dB, Ce, b_layout="col")  # eager, on the same inputs
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int16), Ce.view(torch.int16)), f"replay {rep} differs from the eager call"
    A_last = dA.cpu()
    cref, S = oracle.gemm(FMT["bf16"], A_last, B, oracle.B_NK)
    ok, r, idx = ochk.check(C.float().cpu().double().numpy(), cref, S, K, "bf16")
    assert ok, (r, idx)
