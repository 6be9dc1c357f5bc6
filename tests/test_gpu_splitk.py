"""GPU parity of tg_gemm_ex: the dense GEMM with a caller workspace, which
splits K over several workgroups per output tile where the plan finds that
faster (shapes with few output tiles against a long K).

Each split workgroup stores an fp32 partial tile in the workspace; the last
one to finish adds them in split order and stores C.  Checked here: every
output element against the oracle's bound, bit-identical repeated calls (the
split order is fixed), the workspace's 64 KiB of arrival counters all zero
again after every call (one workspace then serves calls of every shape in
turn), and the workspace-free call agreeing within the bound.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import check as ochk

pytestmark = pytest.mark.gpu

FMT = {"f16": oracle.F16, "bf16": oracle.BF16, "fp8": oracle.E4M3}
TDT = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
ODT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def tg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tile_level_gemm_02_amd as tg

    return tg


def _inputs(dt, M, N, K, lay, seed):
    if dt == "fp8":
        A, sa = synth.quantize_e4m3(synth.normal((M, K), seed))
        B, sb = synth.quantize_e4m3(synth.normal((N, K) if lay == "col" else (K, N), seed + 1))
        return A, B, sa, sb
    A = synth.normal((M, K), seed).to(TDT[dt])
    B = synth.normal((N, K) if lay == "col" else (K, N), seed + 1, std=0.05).to(TDT[dt])
    return A, B, 1.0, 1.0


COUNTER_WORDS = 65536 // 4  # the workspace's arrival counters (include/tg.h)
_SHARED = {}


def _shared_workspace(nbytes):
    """One workspace reused by every case of a test, grown when needed (zeroed once)."""
    ws = _SHARED.get("ws")
    if ws is None or ws.numel() * 4 < nbytes:
        ws = _workspace(nbytes)
        _SHARED["ws"] = ws
    return ws


def _workspace(nbytes):
    """Zeroed device workspace of at least nbytes (256-byte aligned: torch's allocator)."""
    ws = torch.zeros(max(nbytes, 256) // 4 + 64, dtype=torch.int32, device="cuda")
    assert ws.data_ptr() % 256 == 0
    return ws


def _dev(t):
    """t on the GPU with its leading dimension padded to whole 16-byte rows."""
    per = 16 // t.element_size()
    store = torch.zeros((t.shape[0], (t.shape[1] + per - 1) // per * per), dtype=t.dtype, device="cuda")
    store[:, : t.shape[1]] = t.to("cuda")
    return store[:, : t.shape[1]]


def _run(tg, A, B, lay, out, sa, sb, ws):
    M, N = A.shape[0], (B.shape[1] if lay == "row" else B.shape[0])
    C = torch.full((M, (N + 7) // 8 * 8), float("nan"), dtype=ODT[out], device="cuda")[:, :N]
    tg.tg_gemm_ex(_dev(A), _dev(B), C, b_layout=lay, scale_a=sa, scale_b=sb, workspace=ws)
    torch.cuda.synchronize()
    return C


# Shapes the plan splits (few tiles of the chosen edge against a long K):
# rows just past the skinny bound, ragged rows and columns on every tile
# edge, K tails and K step counts that the split count does not divide.
SPLIT_SHAPES = [(33, 2056, 4096), (64, 1024, 8192), (100, 1000, 6144), (130, 2048, 4104), (256, 4096, 4096),
                (300, 1288, 8192), (520, 2048, 3072), (1024, 2048, 8192)]


@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dt,lay,out", [("bf16", "col", "bf16"), ("f16", "row", "f16"), ("fp8", "col", "bf16"),
                                        ("bf16", "row", "f32"), ("fp8", "row", "f32")])
def test_split_parity(tg, dt, lay, out, shape):
    M, N, K = shape
    need = tg.tg_gemm_ex_workspace_bytes(TDT[dt], M, N, K, lay)
    A, B, sa, sb = _inputs(dt, M, N, K, lay, seed=M + N + K)
    ws = _shared_workspace(need)  # (left by earlier cases of other shapes: its counters must be zero)
    C = _run(tg, A, B, lay, out, sa, sb, ws)
    assert int(ws[:COUNTER_WORDS].count_nonzero()) == 0, "the call left the workspace counters non-zero"
    cref, S = oracle.gemm(FMT[dt], A, B, oracle.B_KN if lay == "row" else oracle.B_NK, sa, sb)
    ok, r, idx = ochk.check(C.float().cpu().double().numpy(), cref, S, K, out)
    assert ok, (need, r, idx)
    C2 = _run(tg, A, B, lay, out, sa, sb, ws)
    assert torch.equal(C.view(torch.int16) if out != "f32" else C, C2.view(torch.int16) if out != "f32" else C2), \
        "repeated split calls differ"


def test_split_plans_exist(tg):
    """The shapes above really take a split plan (a positive workspace), and
    the headline shape does not."""
    for M, N, K in [(256, 8192, 8192), (64, 1024, 8192), (33, 2056, 4096)]:
        assert tg.tg_gemm_ex_workspace_bytes(torch.bfloat16, M, N, K) > 0
    assert tg.tg_gemm_ex_workspace_bytes(torch.bfloat16, 4096, 4096, 4096) == 0


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_split_one_hot_exact(tg, dt):
    """One-hot rows of A with a split plan: each output sums one nonzero
    product and zeros from every other split, so C equals B's entries."""
    M, N, K = 256, 2048, 8192
    need = tg.tg_gemm_ex_workspace_bytes(TDT[dt], M, N, K)
    assert need > 0
    Bs = _inputs(dt, 1, N, K, "col", seed=5)[1]
    ks = torch.randint(0, K, (M,), generator=torch.Generator().manual_seed(6))
    A = torch.zeros((M, K))
    A[torch.arange(M), ks] = 1.0
    C = _run(tg, A.to(TDT[dt]), Bs, "col", "f32", 1.0, 1.0, _workspace(need))
    assert torch.equal(C.cpu(), Bs.float().t()[ks])


# More than one round of 256 x 256 tiles with a short last round of 65 to
# 128 tiles and 16-bit inputs: the plan runs the full round's tiles whole and
# splits K only for the last round's tiles (its workspace covers those
# alone), in one launch.  Ragged M, N and K (a partial last K step), both
# layouts of B.  (With fewer tiles left over, or fp8 inputs, the plan runs
# the last round as parts of a second launch instead, without a workspace.)
def _last_round(M, N):
    tiles = ((M + 255) // 256) * ((N + 255) // 256)
    return tiles, tiles - tiles // 256 * 256


def _expect_last_round_split(tg, dt, M, N, K, lay):
    tiles, R = _last_round(M, N)
    assert tiles > 256 and 64 < R <= 128
    need = tg.tg_gemm_ex_workspace_bytes(TDT[dt], M, N, K, lay)
    per_split_tile = 256 * 256 * 4
    assert need > 0 and (need - 65536) % (R * per_split_tile) == 0, "expected the last round's tiles split"
    splits = (need - 65536) // (R * per_split_tile)
    assert 2 <= splits and R * splits <= 256
    print(f"{dt} {M}x{N}x{K} {lay}: {tiles} tiles, last round {R} tiles split {splits} ways", flush=True)
    return need


def test_last_round_split_parity(tg):
    """Every element against the oracle's bound, a bit-identical repeat, and
    the counters left zero."""
    M, N, K = 4400, 4500, 4104
    need = _expect_last_round_split(tg, "bf16", M, N, K, "col")
    A, B, _, _ = _inputs("bf16", M, N, K, "col", seed=41)
    ws = _shared_workspace(need)
    C = _run(tg, A, B, "col", "bf16", 1.0, 1.0, ws)
    assert int(ws[:COUNTER_WORDS].count_nonzero()) == 0
    C2 = _run(tg, A, B, "col", "bf16", 1.0, 1.0, ws)
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16)), "repeated calls differ"
    cref, S = oracle.gemm(oracle.BF16, A, B, oracle.B_NK)
    ok, r, idx = ochk.check(C.float().cpu().double().numpy(), cref, S, K, "bf16")
    assert ok, (r, idx)


@pytest.mark.parametrize("dt,lay,shape", [("bf16", "col", (4400, 4500, 4104)), ("f16", "row", (4400, 4504, 4104)),
                                          ("bf16", "row", (4400, 4504, 8192))],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_last_round_split_one_hot_exact(tg, dt, lay, shape):
    """One-hot rows of A: each output of every tile, whole or split, sums one
    nonzero product and zeros, so C equals B's entries exactly; a tile or a
    K range mapped wrongly shows up as a wrong or missing entry."""
    M, N, K = shape
    need = _expect_last_round_split(tg, dt, M, N, K, lay)
    Bs = _inputs(dt, 1, N, K, lay, seed=43)[1]
    ks = torch.randint(0, K, (M,), generator=torch.Generator().manual_seed(44))
    ks[:4] = torch.tensor([0, K - 1, K // 2, K // 2 - 1])
    A = torch.zeros((M, K))
    A[torch.arange(M), ks] = 1.0
    ws = _shared_workspace(need)
    C = _run(tg, A.to(TDT[dt]), Bs, lay, "f32", 1.0, 1.0, ws)
    assert int(ws[:COUNTER_WORDS].count_nonzero()) == 0
    ref = Bs.float().t()[ks] if lay == "col" else Bs.float()[ks]
    assert torch.equal(C.cpu(), ref)


def test_workspace_free_call_agrees(tg):
    """With no workspace tg_gemm_ex is the plain entry point, bit for bit;
    with one it agrees within the bound."""
    M, N, K = 256, 8192, 8192
    A, B, _, _ = _inputs("bf16", M, N, K, "col", seed=8)
    C0 = _run(tg, A, B, "col", "bf16", 1.0, 1.0, None)
    Cp = torch.empty_like(C0)
    tg.tg_gemm_bf16(A.cuda(), B.cuda(), Cp, b_layout="col")
    torch.cuda.synchronize()
    assert torch.equal(C0.view(torch.int16), Cp.view(torch.int16))
    need = tg.tg_gemm_ex_workspace_bytes(torch.bfloat16, M, N, K)
    assert need > 0
    Cs = _run(tg, A, B, "col", "bf16", 1.0, 1.0, _workspace(need))
    cref, S = oracle.gemm(oracle.BF16, A, B, oracle.B_NK)
    for C in (C0, Cs):
        ok, r, idx = ochk.check(C.float().cpu().double().numpy(), cref, S, K, "bf16")
        assert ok, (r, idx)


def test_workspace_errors(tg):
    M, N, K = 256, 8192, 8192
    A, B, _, _ = _inputs("bf16", M, N, K, "col", seed=9)
    need = tg.tg_gemm_ex_workspace_bytes(torch.bfloat16, M, N, K)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    small = torch.zeros((need - 256) // 4, dtype=torch.int32, device="cuda")
    with pytest.raises(tg.TGError) as e:
        tg.tg_gemm_ex(A.cuda(), B.cuda(), C, workspace=small)
    assert e.value.code == tg.TG_ERR_INVALID_VALUE
    big = torch.zeros(need // 4 + 64, dtype=torch.int32, device="cuda")
    with pytest.raises(tg.TGError) as e:
        tg.tg_gemm_ex(A.cuda(), B.cuda(), C, workspace=big[1:])  # 4-byte offset: misaligned
    assert e.value.code == tg.TG_ERR_MISALIGNED


# The skinny kernel (at most 32 rows against a K-contiguous B) on narrow N:
# with a workspace its split over workgroups goes through partial tiles and
# the last arrival stores C, for every output type (the plain entry point
# splits only fp32 outputs, by atomic adds into a zeroed C).  Ragged N, K
# tails (K % 64, and a partial 16-byte chunk), a split count that does not
# divide the K stages, and row slices.
SKINNY_SPLIT = [(16, 1024, 8192), (5, 520, 4104), (1, 64, 4160), (3, 40, 8200), (24, 200, 6144), (32, 264, 4101)]


@pytest.mark.parametrize("shape", SKINNY_SPLIT, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dt,out", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32")])
def test_skinny_split_workspace(tg, dt, out, shape):
    M, N, K = shape
    need = tg.tg_gemm_ex_workspace_bytes(TDT[dt], M, N, K)
    assert need > 0, "expected a split plan"
    A, B, _, _ = _inputs(dt, M, N, K, "col", seed=M * 3 + N + K)
    ws = _shared_workspace(need)
    C = _run(tg, A, B, "col", out, 1.0, 1.0, ws)
    assert int(ws[:COUNTER_WORDS].count_nonzero()) == 0
    cref, S = oracle.gemm(FMT[dt], A, B, oracle.B_NK)
    ok, r, idx = ochk.check(C.float().cpu().double().numpy(), cref, S, K, out)
    assert ok, (r, idx)
    C2 = _run(tg, A, B, "col", out, 1.0, 1.0, ws)
    assert torch.equal(C.view(torch.int16) if out != "f32" else C, C2.view(torch.int16) if out != "f32" else C2)


# 33 .. 48 rows against a K-contiguous B: the skinny kernel in row slices,
# unless a caller workspace lets the NT kernel split K.  Where the NT plan
# does not split (too few K steps) tg_gemm_ex with a workspace takes the same
# kernel as the plain entry point, bit for bit; where it splits, the NT
# kernel's result meets the bound.
@pytest.mark.parametrize("shape,nt_splits", [((40, 1000, 256), False), ((48, 264, 448), False),
                                             ((33, 2056, 4096), True), ((48, 1000, 8192), True)],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_skinny_or_split_nt_above_32_rows(tg, shape, nt_splits):
    M, N, K = shape
    need = tg.tg_gemm_ex_workspace_bytes(torch.bfloat16, M, N, K)
    assert (need > 0) == nt_splits
    A, B, _, _ = _inputs("bf16", M, N, K, "col", seed=M + N + K + 11)
    Cx = _run(tg, A, B, "col", "bf16", 1.0, 1.0, _workspace(max(need, 4096)))
    Cp = torch.full_like(Cx, float("nan"))
    tg.tg_gemm_bf16(_dev(A), _dev(B), Cp, b_layout="col")
    torch.cuda.synchronize()
    if not nt_splits:
        assert torch.equal(Cx.view(torch.int16), Cp.view(torch.int16)), "same kernel, different bits"
    cref, S = oracle.gemm(oracle.BF16, A, B, oracle.B_NK)
    for C in (Cx, Cp):
        ok, r, idx = ochk.check(C.float().cpu().double().numpy(), cref, S, K, "bf16")
        assert ok, (r, idx)


# ---------------------------------------------------------------- w4a16
# tg_gemm_w4a16_ex: the 128 x 128 w4a16 kernel with K split over workgroups
# (each dequantised word feeds four MFMAs).  The w4a16 workload itself, and
# ragged rows, columns and K ranges whose split leaves an odd number of
# scale-group pairs per workgroup.

def _w4_inputs(M, N, K, seed):
    A = synth.normal((M, K), seed).to(torch.float16)
    q = synth.random_words((N, K // 8), seed + 1)
    s = synth.uniform((N, K // 128), seed + 2, 0.005, 0.02).to(torch.float16)
    return A, q, s


def _run_w4_ex(tg, A, q, s, ws, zp=8):
    M, N = A.shape[0], q.shape[0]
    C = torch.full((M, (N + 7) // 8 * 8), float("nan"), dtype=torch.float16, device="cuda")[:, :N]
    tg.tg_gemm_w4a16_ex(A.cuda(), q.cuda(), s.cuda(), C, zero_point=zp, workspace=ws)
    torch.cuda.synchronize()
    return C


W4_SPLIT = [(256, 8192, 8192), (100, 1000, 4096), (130, 520, 2560), (64, 1024, 8192), (200, 2056, 3072)]


@pytest.mark.parametrize("zp", [8, 3])
@pytest.mark.parametrize("shape", W4_SPLIT, ids=lambda s: "x".join(map(str, s)))
def test_w4a16_split_parity(tg, shape, zp):
    M, N, K = shape
    need = tg.tg_gemm_w4a16_ex_workspace_bytes(M, N, K)
    assert need > 0, "expected a split plan"
    A, q, s = _w4_inputs(M, N, K, seed=M + N + K + zp)
    ws = _shared_workspace(need)
    C = _run_w4_ex(tg, A, q, s, ws, zp)
    assert int(ws[:COUNTER_WORDS].count_nonzero()) == 0
    cref, S = oracle.w4a16(A, q, s, K, zero_point=zp)
    ok, r, idx = ochk.check(C.float().cpu().double().numpy(), cref, S, K, "f16")
    assert ok, (r, idx)
    C2 = _run_w4_ex(tg, A, q, s, ws, zp)
    assert torch.equal(C.view(torch.int16), C2.view(torch.int16)), "repeated split calls differ"


def test_w4a16_split_one_hot_matches_dequant(tg):
    """One-hot rows of A through the split kernel give tg_dequant_w4's weights bit for bit."""
    M, N, K = 256, 1032, 4096
    need = tg.tg_gemm_w4a16_ex_workspace_bytes(M, N, K)
    assert need > 0
    _, q, s = _w4_inputs(1, N, K, seed=71)
    W = torch.empty((N, K), dtype=torch.float16, device="cuda")
    tg.tg_dequant_w4(q.cuda(), s.cuda(), W, K, zero_point=5)
    ks = torch.randint(0, K, (M,), generator=torch.Generator().manual_seed(72))
    ks[:16] = torch.arange(16) * (K // 16) + torch.arange(16) % 8
    A = torch.zeros((M, K), dtype=torch.float16)
    A[torch.arange(M), ks] = 1.0
    C = _run_w4_ex(tg, A, q, s, _shared_workspace(need), zp=5)
    assert torch.equal(C.cpu().view(torch.int16), W.cpu().t()[ks].view(torch.int16))


def test_w4a16_ex_without_workspace_is_plain(tg):
    M, N, K = 256, 1024, 2048
    A, q, s = _w4_inputs(M, N, K, seed=73)
    C0 = _run_w4_ex(tg, A, q, s, None)
    C1 = torch.empty_like(C0)
    tg.tg_gemm_w4a16(A.cuda(), q.cuda(), s.cuda(), C1)
    torch.cuda.synchronize()
    assert torch.equal(C0.view(torch.int16), C1.view(torch.int16))
