#!/usr/bin/env python3
"""Benchmark of the tile GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-secondary]

A step is one call of the GEMM on the headline workload: bf16 4096^3, A
row-major, B column-major, fp32 accumulate, bf16 out (inputs N(0,1) rounded
to bf16, seeded).  One call runs the whole hot path: output-tile grid,
global->LDS tile copies, MFMA tile products into register accumulators, the
pipelined K loop and the epilogue store.

Before the W warmup steps the headline kernel runs back to back for
SETTLE_S seconds (untimed, reported as `settle_s`): the GPU takes some
20-30 ms of sustained load to reach its clocks, and a handful of warmup
launches would otherwise leave the timed steps on the clock ramp.

Printed: ONE JSON line with the metric, `roofline` (the GEMM kernel's
achieved TFLOP/s against the dense bf16 MFMA peak, from one pair of HIP
events around the K timed launches on their stream), `cpu_baseline` (the CPU oracle timed
on a bounded sample of the same workload) and `secondary` (the skinny M=16
GEMM's GB/s against the HBM peak, the same GEMM on an 8-way column shard
(N=1024), the fp8 and w4a16 workloads, the w4a16 weights at decode batch
sizes M=16 and M=1, the w4a16 workload and bf16 M=256 x 8192 x 8192 with
the split of K over workgroups (tg_gemm_w4a16_ex, tg_gemm_ex) and without, the fp8 workload with B row-major, and the
2:4 sparse GEMM at 4096^3), each
secondary timed launch by launch with the 256 MB Infinity Cache flushed
(by a 512 MiB read) before every launch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s (% MFMA peak) at bf16 4096³; GB/s (% HBM peak) at M=16 skinny"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU, dense
PEAK_FP8_TFLOPS = 5033.2   # x 8192 FLOP/clk/CU, dense
PEAK_HBM_GBS = 8000.0
FLUSH_BYTES = 512 << 20   # > 2x the 256 MB Infinity Cache


def kernel_source_hash() -> str:
    """Hash of the HIP sources: a stored counter reading is valid only for this hash."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tile_level_gemm_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _events(n):
    import torch

    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def time_launches(fn, n: int, flush=None):
    """Per-launch durations (s) from event pairs on the current stream around each call."""
    import torch

    ev = _events(n)
    for i in range(n):
        if flush is not None:
            flush()
        ev[i][0].record()
        fn()
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e-3 for a, b in ev]


def median(xs):
    s = sorted(xs)
    return s[len(s) // 2]


def make_flush():
    """Evict the Infinity Cache by READING 512 MiB (twice its size).

    A write-based flush would leave ~256 MB of dirty lines whose write-back
    then competes with the next kernel's reads (measured: it halves the read
    bandwidth a streaming kernel sees right after it)."""
    import torch

    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    out = torch.empty((), dtype=torch.float32, device="cuda")
    return lambda: torch.sum(buf, dim=0, out=out)


# ------------------------------------------------------------------ workloads

def setup_bf16_4096():
    import torch
    import synth
    import tile_level_gemm_02_amd as tg

    w = synth.workload("bf16_4096")
    A, B = w["A"].cuda(), w["B"].cuda()
    C = torch.empty((w["M"], w["N"]), dtype=torch.bfloat16, device="cuda")
    fn = lambda: tg.tg_gemm_bf16(A, B, C, b_layout="col")
    flops = 2.0 * w["M"] * w["N"] * w["K"]
    bytes_ = 2 * (w["M"] * w["K"] + w["N"] * w["K"] + w["M"] * w["N"])
    return w, fn, flops, bytes_


def setup_skinny():
    import torch
    import synth
    import tile_level_gemm_02_amd as tg

    w = synth.workload("bf16_skinny")
    A, B = w["A"].cuda(), w["B"].cuda()
    C = torch.empty((w["M"], w["N"]), dtype=torch.float32, device="cuda")
    fn = lambda: tg.tg_gemm_bf16(A, B, C, b_layout="col")
    flops = 2.0 * w["M"] * w["N"] * w["K"]
    bytes_ = 2 * (w["M"] * w["K"] + w["N"] * w["K"]) + 4 * w["M"] * w["N"]
    return w, fn, flops, bytes_


def setup_skinny_shard(ws_split: bool = False):
    """The skinny workload's 8-way column shard: M=16, N=1024, K=8192.  The
    plain entry point splits K by atomic adds into a C that a fill kernel
    zeroes first; with a workspace (tg_gemm_ex) the split hands its partial
    tiles to the last arrival and no fill runs."""
    import torch
    import synth
    import tile_level_gemm_02_amd as tg

    w = synth.workload("bf16_skinny", N=1024)
    A, B = w["A"].cuda(), w["B"].cuda()
    C = torch.empty((w["M"], w["N"]), dtype=torch.float32, device="cuda")
    if ws_split:
        need = tg.tg_gemm_ex_workspace_bytes(torch.bfloat16, w["M"], w["N"], w["K"])
        ws = torch.zeros(max(need, 256) // 4, dtype=torch.int32, device="cuda")
        fn = lambda: tg.tg_gemm_ex(A, B, C, b_layout="col", workspace=ws)
    else:
        fn = lambda: tg.tg_gemm_bf16(A, B, C, b_layout="col")
    flops = 2.0 * w["M"] * w["N"] * w["K"]
    bytes_ = 2 * (w["M"] * w["K"] + w["N"] * w["K"]) + 4 * w["M"] * w["N"]
    return w, fn, flops, bytes_


def setup_sp24():
    """2:4 sparse weights at 4096^3: bf16 A, compressed bf16 W (values + codes), bf16 out."""
    import torch
    import synth
    import tile_level_gemm_02_amd as tg

    w = synth.workload("sp24_4096")
    A, v, m = w["A"].cuda(), w["vals"].cuda(), w["meta"].cuda()
    C = torch.empty((w["M"], w["N"]), dtype=torch.bfloat16, device="cuda")
    fn = lambda: tg.tg_gemm_sp24_bf16(A, v, m, C)
    M, N, K = w["M"], w["N"], w["K"]
    flops = 2.0 * M * N * K  # dense-equivalent
    bytes_ = 2 * M * K + N * K + N * K // 8 + 2 * M * N
    return w, fn, flops, bytes_


def setup_bf16_m256(split: bool):
    """bf16 M=256, N=K=8192 (a few hundred rows against a large weight), bf16 out:
    the plain entry point, or tg_gemm_ex with a workspace (K split over workgroups)."""
    import torch
    import synth
    import tile_level_gemm_02_amd as tg

    w = synth.workload("bf16_4096", M=256, N=8192, K=8192)
    A, B = w["A"].cuda(), w["B"].cuda()
    C = torch.empty((w["M"], w["N"]), dtype=torch.bfloat16, device="cuda")
    if split:
        need = tg.tg_gemm_ex_workspace_bytes(torch.bfloat16, w["M"], w["N"], w["K"])
        ws = torch.zeros(max(need, 256) // 4, dtype=torch.int32, device="cuda")
        fn = lambda: tg.tg_gemm_ex(A, B, C, b_layout="col", workspace=ws)
    else:
        fn = lambda: tg.tg_gemm_bf16(A, B, C, b_layout="col")
    M, N, K = w["M"], w["N"], w["K"]
    return w, fn, 2.0 * M * N * K, 2 * (M * K + N * K + M * N)


def setup_bf16_4608(split: bool):
    """bf16 4608^3 (324 tiles of 256 x 256: a second round of 68 tiles on 256
    compute units), bf16 out: the plain entry point, or tg_gemm_ex with a
    workspace (the last round's tiles split K behind the whole ones)."""
    import torch
    import synth
    import tile_level_gemm_02_amd as tg

    w = synth.workload("bf16_4096", M=4608, N=4608, K=4608)
    A, B = w["A"].cuda(), w["B"].cuda()
    C = torch.empty((w["M"], w["N"]), dtype=torch.bfloat16, device="cuda")
    if split:
        need = tg.tg_gemm_ex_workspace_bytes(torch.bfloat16, w["M"], w["N"], w["K"])
        ws = torch.zeros(max(need, 256) // 4, dtype=torch.int32, device="cuda")
        fn = lambda: tg.tg_gemm_ex(A, B, C, b_layout="col", workspace=ws)
    else:
        fn = lambda: tg.tg_gemm_bf16(A, B, C, b_layout="col")
    M, N, K = w["M"], w["N"], w["K"]
    return w, fn, 2.0 * M * N * K, 2 * (M * K + N * K + M * N)


def setup_fp8_rowb():
    """The fp8 workload with B stored row-major (K x N): transposing LDS reads."""
    import torch
    import synth
    import tile_level_gemm_02_amd as tg

    w = synth.workload("fp8_8192")
    A, B = w["A"].cuda(), w["B"].t().contiguous().cuda()
    C = torch.empty((w["M"], w["N"]), dtype=torch.bfloat16, device="cuda")
    fn = lambda: tg.tg_gemm_fp8(A, B, C, w["scale_a"], w["scale_b"], b_layout="row")
    flops = 2.0 * w["M"] * w["N"] * w["K"]
    bytes_ = w["M"] * w["K"] + w["N"] * w["K"] + 2 * w["M"] * w["N"]
    return w, fn, flops, bytes_


def setup_fp8():
    import torch
    import synth
    import tile_level_gemm_02_amd as tg

    w = synth.workload("fp8_8192")
    A, B = w["A"].cuda(), w["B"].cuda()
    C = torch.empty((w["M"], w["N"]), dtype=torch.bfloat16, device="cuda")
    fn = lambda: tg.tg_gemm_fp8(A, B, C, w["scale_a"], w["scale_b"], b_layout="col")
    flops = 2.0 * w["M"] * w["N"] * w["K"]
    bytes_ = w["M"] * w["K"] + w["N"] * w["K"] + 2 * w["M"] * w["N"]
    return w, fn, flops, bytes_


def setup_w4a16(M=None, split=False):
    """The w4a16 workload (M rows); with split, tg_gemm_w4a16_ex with a workspace (K split over workgroups)."""
    import torch
    import synth
    import tile_level_gemm_02_amd as tg

    w = synth.workload("w4a16", M=M)
    A, q, s = w["A"].cuda(), w["qweight"].cuda(), w["scales"].cuda()
    C = torch.empty((w["M"], w["N"]), dtype=torch.float16, device="cuda")
    if split:
        need = tg.tg_gemm_w4a16_ex_workspace_bytes(w["M"], w["N"], w["K"])
        ws = torch.zeros(max(need, 256) // 4, dtype=torch.int32, device="cuda")
        fn = lambda: tg.tg_gemm_w4a16_ex(A, q, s, C, workspace=ws)
    else:
        fn = lambda: tg.tg_gemm_w4a16(A, q, s, C)
    M, N, K = w["M"], w["N"], w["K"]
    flops = 2.0 * M * N * K
    bytes_ = 2 * M * K + N * K // 2 + 2 * N * (K // 128) + 2 * M * N
    return w, fn, flops, bytes_


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(target_seconds: float = 12.0):
    """The oracle (fp64, host threads) on a bounded row sample of the bf16 4096^3 workload."""
    import oracle
    import synth

    w = synth.workload("bf16_4096")
    cores = len(os.sched_getaffinity(0))  # every core this process may run on
    # time two small row samples, fit t = t0 + rows * per_row, size the sample for ~target_seconds
    def run(r):
        t0 = time.perf_counter()
        oracle.gemm(oracle.BF16, w["A"][:r], w["B"], oracle.B_NK, nthreads=cores)
        return time.perf_counter() - t0

    r1, r2 = cores, 4 * cores
    t1, t2 = run(r1), run(r2)
    per_row = max((t2 - t1) / (r2 - r1), 1e-6)
    rows2 = int(min(w["M"], max(r2, (target_seconds - max(t1 - r1 * per_row, 0.0)) / per_row)))
    rows2 = max(cores, rows2 // cores * cores)
    dt = run(rows2)
    flops = 2.0 * rows2 * w["N"] * w["K"]
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{rows2} of {w['M']} rows of the bf16 4096^3 product (fp64 triple loop incl. "
                      f"decode of B), {dt:.1f} s on {cores} threads"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------------ main

SETTLE_S = 0.2  # untimed back-to-back headline launches before the warmup steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed launches first: the GPU takes some 20-30 ms of sustained load to reach its clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--back-to-back", action="store_true",
                    help="with --only: no cache flush between the launches (sustained load, e.g. to sample clocks)")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="only run plain device-to-device copies of MIB MiB (to scale HBM byte counters)")
    ap.add_argument("--only", choices=["bf16_4096", "bf16_skinny", "bf16_skinny_n1024", "bf16_skinny_n1024_ws", "fp8_8192", "fp8_8192_rowb",
                                       "w4a16", "w4a16_split", "w4a16_m16", "w4a16_m1", "sp24_4096", "bf16_m256",
                                       "bf16_m256_split"],
                    default=None,
                    help="only run this workload's launches (for counter collection), no JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library and this benchmark run on one GPU; --gpus {args.gpus} is not supported "
              "(over several GPUs the GEMM would shard by output columns, with no exchange between them)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibrate:
        n = args.copy_calibrate << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch_read": n, "copy_bytes_per_launch_written": n,
                          "launches": args.steps}), flush=True)
        return
    flush = make_flush()
    flush()  # its first call loads the reduction kernel (≈24 ms): not between the warm-up and the timed steps
    torch.cuda.synchronize()
    if args.only:
        setup = {"bf16_4096": setup_bf16_4096, "bf16_skinny": setup_skinny, "bf16_skinny_n1024": setup_skinny_shard,
                 "bf16_skinny_n1024_ws": lambda: setup_skinny_shard(True), "fp8_8192": setup_fp8, "fp8_8192_rowb": setup_fp8_rowb,
                 "bf16_m256": lambda: setup_bf16_m256(False), "bf16_m256_split": lambda: setup_bf16_m256(True),
                 "w4a16": setup_w4a16, "w4a16_split": lambda: setup_w4a16(split=True), "w4a16_m16": lambda: setup_w4a16(16), "sp24_4096": setup_sp24,
                 "w4a16_m1": lambda: setup_w4a16(1)}[args.only]
        _, fn, _, _ = setup()
        for _ in range(args.warmup):
            fn()
        for _ in range(args.steps):
            if not args.back_to_back:
                flush()
            fn()
        torch.cuda.synchronize()
        return

    # ---- headline: bf16 4096^3
    w, fn, flops, nbytes = setup_bf16_4096()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < SETTLE_S:  # clocks up before the warmup steps
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        fn()
    flush()  # inputs start the timed region in HBM, not in the Infinity Cache
    # one event pair around the K back-to-back launches (on the stream they are
    # issued to): events between launches would separate the kernels
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch = e0.elapsed_time(e1) * 1e-3 / args.steps
    ms_per_step = wall / args.steps * 1e3
    value = flops / (wall / args.steps) / 1e12
    achieved = flops / avg_launch / 1e12


    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rounded to bf16)",
        "config": {"workload": "bf16 GEMM M=N=K=4096, A row-major, B column-major, fp32 accumulate, bf16 out",
                   "M": 4096, "N": 4096, "K": 4096, "b_layout": "col", "out": "bf16"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": stored_traffic("bf16_4096"),
                     "kernel": "gemm_nt<bf16, bf16 out, 256x256 tile, 8 waves, 2 LDS stages of 128 B rows>",
                     "flop_per_launch": flops, "avg_launch_us": round(avg_launch * 1e6, 3)},
    }

    # ---- secondary workloads, each launch preceded by an Infinity Cache flush
    if not args.no_secondary:
        sec = {}
        n = max(10, min(args.steps, 50))
        for name, setup, peak_key in (("bf16_skinny", setup_skinny, "hbm"), ("bf16_skinny_n1024", setup_skinny_shard, "hbm"),
                                      ("bf16_skinny_n1024_ws", lambda: setup_skinny_shard(True), "hbm"),
                                      ("fp8_8192", setup_fp8, "fp8"),
                                      ("w4a16", setup_w4a16, "both"),
                                      ("w4a16_split", lambda: setup_w4a16(split=True), "both"),
                                      ("w4a16_m16", lambda: setup_w4a16(16), "hbm"),
                                      ("w4a16_m1", lambda: setup_w4a16(1), "hbm"),
                                      ("bf16_m256", lambda: setup_bf16_m256(False), "mfma"),
                                      ("bf16_m256_split", lambda: setup_bf16_m256(True), "mfma"),
                                      ("bf16_4608", lambda: setup_bf16_4608(False), "mfma"),
                                      ("bf16_4608_split", lambda: setup_bf16_4608(True), "mfma"),
                                      ("fp8_8192_rowb", setup_fp8_rowb, "fp8"),
                                      ("sp24_4096", setup_sp24, "sp")):
            w2, fn2, fl2, by2 = setup()
            for _ in range(3):
                fn2()
            ts = time_launches(fn2, n if not name.startswith("fp8_8192") else max(10, n // 2), flush=flush)
            t = median(ts)
            rec = {"median_us": round(t * 1e6, 3), "min_us": round(min(ts) * 1e6, 3),
                   "TFLOP/s": round(fl2 / t / 1e12, 2), "GB/s": round(by2 / t / 1e9, 1),
                   "hbm_frac": round(by2 / t / 1e9 / PEAK_HBM_GBS, 4),
                   "algorithmic_bytes": by2, "flop": fl2}
            if peak_key == "fp8":
                rec["mfma_frac"] = round(fl2 / t / 1e12 / PEAK_FP8_TFLOPS, 4)
            elif peak_key == "sp":  # dense-equivalent FLOP against the 2:4 sparse rate (twice dense bf16)
                rec["mfma_frac"] = round(fl2 / t / 1e12 / (2 * PEAK_BF16_TFLOPS), 4)
            else:
                rec["mfma_frac"] = round(fl2 / t / 1e12 / PEAK_BF16_TFLOPS, 4)
            sec[name] = rec
            del fn2
            torch.cuda.empty_cache()
        out["secondary"] = sec

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
