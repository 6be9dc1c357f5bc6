"""Calls captured in a HIP graph and replayed: the library launches only
kernels (no allocation, memset or copy), so a captured call replays the same
plan on whatever the input buffers then hold.  Covered: a split plan with a
caller workspace (partial tiles and arrival counters that must return to
zero for the next replay), a plan of two launches (a short last round cut
into smaller tiles), the skinny kernel's fp32 atomic split (a fill kernel,
then atomic adds) and the w4a16 split.  Each replay follows new contents of
A, with eager calls and synchronizations in between; a deterministic plan
must equal the eager call bit for bit, and the atomic one (its summation
order varies) must meet the oracle's bound."""
import pytest
import torch

import oracle
import synth
from oracle import check as ochk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_gemm_02_amd as tg

    return tg


def _bits(t):
    return t if t.dtype == torch.float32 else t.view(torch.int16)


def _replay(tg, make_call, A_shape, A_dtype, out_shape, out_dtype, seed, exact=True, check=None):
    dA = torch.empty(A_shape, dtype=A_dtype, device="cuda")
    C = torch.full(out_shape, float("nan"), dtype=out_dtype, device="cuda")
    Ce = torch.empty_like(C)
    dA.copy_(synth.normal(A_shape, seed).to(A_dtype))
    call = make_call(dA)
    call(Ce)  # eager first: anything set up on a first call happens outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(C)
    torch.cuda.synchronize()
    for rep in range(3):
        print(f"replay {rep}", flush=True)
        A = synth.normal(A_shape, seed + 1 + rep).to(A_dtype)
        dA.copy_(A)
        call(Ce)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if exact:
            assert torch.equal(_bits(C), _bits(Ce)), f"replay {rep} differs from the eager call"
        else:
            check(A, C)


def test_graph_split_with_workspace(tg):
    M, N, K = 4400, 4504, 4104  # a last round of 68 tiles split over K
    B = synth.normal((N, K), 11, std=0.05).to(torch.bfloat16).cuda()
    need = tg.tg_gemm_ex_workspace_bytes(torch.bfloat16, M, N, K)
    assert need > 0
    ws = torch.zeros(need // 4 + 64, dtype=torch.int32, device="cuda")

    def make(dA):
        return lambda C: tg.tg_gemm_ex(dA, B, C, b_layout="col", workspace=ws)

    _replay(tg, make, (M, K), torch.bfloat16, (M, N), torch.bfloat16, seed=10)
    assert int(ws[: 65536 // 4].count_nonzero()) == 0


def test_graph_two_launch_plan(tg):
    M, N, K = 4300, 4000, 1032  # 17 x 16 tiles of 256: a last round of 16 cut into 64 x 64 parts
    B = synth.normal((N, K), 21, std=0.05).to(torch.float16).cuda()

    def make(dA):
        return lambda C: tg.tg_gemm_f16(dA, B, C, b_layout="col")

    _replay(tg, make, (M, K), torch.float16, (M, N), torch.float32, seed=20)


def test_graph_skinny_atomic_split(tg):
    M, N, K = 16, 1024, 8192  # fp32 output without a workspace: K split by atomic adds
    Bh = synth.normal((N, K), 31, std=0.05).to(torch.bfloat16)
    B = Bh.cuda()

    def make(dA):
        return lambda C: tg.tg_gemm_bf16(dA, B, C, b_layout="col")

    def check(A, C):
        cref, S = oracle.gemm(oracle.BF16, A, Bh, oracle.B_NK)
        ok, r, idx = ochk.check(C.cpu().double().numpy(), cref, S, K, "f32")
        assert ok, (r, idx)

    _replay(tg, make, (M, K), torch.bfloat16, (M, N), torch.float32, seed=30, exact=False, check=check)


def test_graph_w4a16_split(tg):
    M, N, K = 256, 8192, 8192
    q = synth.random_words((N, K // 8), 41).cuda()
    s = synth.uniform((N, K // 128), 42, 0.005, 0.02).to(torch.float16).cuda()
    need = tg.tg_gemm_w4a16_ex_workspace_bytes(M, N, K)
    assert need > 0
    ws = torch.zeros(need // 4 + 64, dtype=torch.int32, device="cuda")

    def make(dA):
        return lambda C: tg.tg_gemm_w4a16_ex(dA, q, s, C, workspace=ws)

    _replay(tg, make, (M, K), torch.float16, (M, N), torch.float16, seed=40)
