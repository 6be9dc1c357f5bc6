"""CPU sanitizer runs (AddressSanitizer + UndefinedBehaviorSanitizer).

* The oracle: oracle/oracle.c with tests/sanitize/oracle_driver.c, built by
  gcc with -fsanitize=address,undefined, every buffer at its exact extent.
* The host side of the library: every tile_level_gemm_02_amd/csrc/*.hip
  compiled for the host only (the device pass is skipped, so no GPU code is
  built or run) with the sanitizers on the host pass, linked with
  tests/sanitize/abi_driver.cpp, which calls every entry point with arguments
  that fail validation, empty problems and a grid of workspace-size queries up
  to INT64_MAX.  A host-only object refers to its device code by a symbol the
  device link would define; an empty offload bundle stands in for it (no
  kernel is launched, so the HIP runtime never reads it).

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), which
fails the test with the report."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", *SAN, "-pthread",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_library_host_path_under_asan_ubsan(tmp_path):
    host = ["-Xarch_host"]
    flags = ["--offload-arch=gfx950", "--offload-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Wno-unused-command-line-argument", "-w", "-I", os.path.join(ROOT, "include")]
    for f in SAN:
        flags += host + [f]
    srcs = sorted(glob.glob(os.path.join(ROOT, "tile_level_gemm_02_amd", "csrc", "*.hip")))
    srcs.append(os.path.join(HERE, "abi_driver.cpp"))

    def cc(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        _run([HIPCC, *flags, *lang, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(cc, srcs))
    # the device-code symbols the host-only objects refer to: empty offload bundles
    syms = set()
    for o in objs:
        out = _run(["nm", "-u", o]).stdout
        syms.update(line.split()[-1] for line in out.splitlines() if "__hip_fatbin_" in line)
    stub = tmp_path / "fatbin_stub.c"
    stub.write_text("".join(f'__attribute__((aligned(4096))) const char {s}[32] = "__CLANG_OFFLOAD_BUNDLE__";\n'
                            for s in sorted(syms)))
    stub_o = str(tmp_path / "fatbin_stub.o")
    _run(["gcc", "-c", str(stub), "-o", stub_o])
    exe = str(tmp_path / "abi_asan")
    link = [HIPCC, "--offload-arch=gfx950", "--offload-host-only"]
    for f in SAN[:1]:
        link += host + [f]
    _run([*link, *objs, stub_o, "-o", exe])
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.strip() == "ok", r.stdout + r.stderr
