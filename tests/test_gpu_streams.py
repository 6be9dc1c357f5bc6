"""Calls in flight together on several streams of one GPU, each with its own
workspace, do not interfere: the library keeps no state between calls apart
from the static scratch of tg_gemm_ex_noalloc, which is not used here.  Split
plans (partial tiles and arrival counters in the workspace), a plain plan and
a w4a16 split run concurrently on four streams, several times each.  Every
result must equal the same call made alone on the default stream bit for bit,
and every workspace's arrival counters must be zero again at the end."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

TDT = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
COUNTER_WORDS = 65536 // 4

# (input, output, M, N, K): a last round of 68 tiles split over K, every
# tile split, the skinny kernel's split, an fp8 split, a plain plan
DENSE = [("bf16", torch.bfloat16, 4400, 4504, 4104), ("bf16", torch.bfloat16, 256, 8192, 8192),
         ("f16", torch.float32, 24, 1024, 8192), ("fp8", torch.bfloat16, 40, 1000, 4096),
         ("bf16", torch.float32, 2048, 2048, 1024)]


@pytest.fixture(scope="module")
def tg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_gemm_02_amd as tg

    return tg


def _dense_job(tg, i, dt, odt, M, N, K):
    if dt == "fp8":
        A, sa = synth.quantize_e4m3(synth.normal((M, K), 50 + i))
        B, sb = synth.quantize_e4m3(synth.normal((N, K), 60 + i))
    else:
        A, sa = synth.normal((M, K), 50 + i).to(TDT[dt]), 1.0
        B, sb = synth.normal((N, K), 60 + i, std=0.05).to(TDT[dt]), 1.0
    dA, dB = A.cuda(), B.cuda()
    need = tg.tg_gemm_ex_workspace_bytes(TDT[dt], M, N, K)

    def run(C, ws, stream=None):
        tg.tg_gemm_ex(dA, dB, C, b_layout="col", scale_a=sa, scale_b=sb, workspace=ws, stream=stream)

    return run, (M, N), odt, need


def _w4_job(tg):
    M, N, K = 256, 8192, 8192
    A = synth.normal((M, K), 70).to(torch.float16).cuda()
    q = synth.random_words((N, K // 8), 71).cuda()
    s = synth.uniform((N, K // 128), 72, 0.005, 0.02).to(torch.float16).cuda()
    need = tg.tg_gemm_w4a16_ex_workspace_bytes(M, N, K)

    def run(C, ws, stream=None):
        tg.tg_gemm_w4a16_ex(A, q, s, C, workspace=ws, stream=stream)

    return run, (M, N), torch.float16, need


def _bits(t):
    return t if t.dtype == torch.float32 else t.view(torch.int16)


def test_concurrent_streams_match_sequential(tg):
    jobs = [_dense_job(tg, i, *c) for i, c in enumerate(DENSE)] + [_w4_job(tg)]
    assert sum(1 for j in jobs if j[3] > 0) >= 5, "expected split plans"
    ref = []
    for run, shape, odt, need in jobs:  # alone, on the default stream
        C = torch.full(shape, float("nan"), dtype=odt, device="cuda")
        ws = torch.zeros(max(need, 256) // 4 + 64, dtype=torch.int32, device="cuda")
        run(C, ws)
        torch.cuda.synchronize()
        ref.append(C)
    streams = [torch.cuda.Stream() for _ in range(4)]
    outs = [[torch.full(shape, float("nan"), dtype=odt, device="cuda") for _ in range(3)]
            for _, shape, odt, _ in jobs]
    wss = [torch.zeros(max(need, 256) // 4 + 64, dtype=torch.int32, device="cuda") for _, _, _, need in jobs]
    torch.cuda.synchronize()
    for rep in range(3):  # job j on stream (j + rep) % 4: every stream carries several plans at once
        for j, (run, _, _, _) in enumerate(jobs):
            st = streams[(j + rep) % len(streams)]
            with torch.cuda.stream(st):
                # the job's workspace is reused on another stream next repeat
                if rep:
                    st.wait_stream(streams[(j + rep - 1) % len(streams)])
                run(outs[j][rep], wss[j], stream=st)
    torch.cuda.synchronize()
    for j in range(len(jobs)):
        for rep in range(3):
            assert torch.equal(_bits(outs[j][rep]), _bits(ref[j])), f"job {j} repeat {rep} differs from the lone call"
        assert int(wss[j][:COUNTER_WORDS].count_nonzero()) == 0, f"job {j} left its workspace counters non-zero"
