"""The C-ABI library: it loads, exports every declared symbol, and rejects
invalid arguments before any HIP call (CPU only: nothing here launches)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "tg.h")).read()
    return sorted(set(re.findall(r"\b(tg_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def tg():
    import tile_level_gemm_02_amd as tg

    return tg


def test_header_declares_expected_entry_points():
    assert _declared() == sorted(["tg_gemm_f16", "tg_gemm_bf16", "tg_gemm_fp8", "tg_gemm_w4a16",
                                  "tg_dequant_w4", "tg_gemm_sp24_bf16", "tg_gemm_ex", "tg_gemm_ex_workspace_bytes",
                                  "tg_gemm_ex_noalloc", "tg_gemm_w4a16_ex", "tg_gemm_w4a16_ex_workspace_bytes",
                                  "tg_status_string", "tg_version"])


def test_library_exports_every_declared_symbol(tg):
    lib = ctypes.CDLL(tg.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(tg.EXPORTS)


def test_status_strings(tg):
    for code in range(6):
        s = tg.tg_status_string(code)
        assert s.startswith("TG_")
    assert "unknown" in tg.tg_status_string(99)
    assert tg.tg_version() == 100


A16 = 0x10000  # a fake, 16-byte aligned "device" address: never dereferenced on these paths


def _dense(lib, fn, M=8, N=8, K=8, A=A16, lda=8, B=A16, ldb=8, lay=0, C=A16, ldc=8, cd=0):
    return getattr(lib, fn)(M, N, K, A, lda, B, ldb, lay, C, ldc, cd, None)


@pytest.mark.parametrize("fn", ["tg_gemm_f16", "tg_gemm_bf16"])
def test_dense_validation(tg, fn):
    lib = tg.lib
    E = dict(inv=tg.TG_ERR_INVALID_VALUE, mis=tg.TG_ERR_MISALIGNED)
    assert _dense(lib, fn, M=-1) == E["inv"]
    assert _dense(lib, fn, K=-3) == E["inv"]
    assert _dense(lib, fn, lay=2) == E["inv"]
    assert _dense(lib, fn, cd=7) == E["inv"]
    assert _dense(lib, fn, A=None) == E["inv"]
    assert _dense(lib, fn, C=None) == E["inv"]
    assert _dense(lib, fn, lda=7) == E["inv"]        # lda < K
    assert _dense(lib, fn, ldc=4) == E["inv"]        # ldc < N
    assert _dense(lib, fn, N=16, ldb=8, lay=0) == E["inv"]  # row-major B needs ldb >= N
    assert _dense(lib, fn, K=4, lda=12) == E["mis"]  # 24 bytes per row
    assert _dense(lib, fn, A=A16 + 8) == E["mis"]
    assert _dense(lib, fn, C=A16 + 4) == E["mis"]
    assert _dense(lib, fn, ldc=12, cd=1) == E["mis"]  # 24-byte fp16 rows
    # empty problems are a successful no-op, whatever the pointers
    assert _dense(lib, fn, M=0, A=None, B=None, C=None) == tg.TG_OK
    assert _dense(lib, fn, N=0, A=None, B=None, C=None) == tg.TG_OK


def test_fp8_validation(tg):
    lib = tg.lib
    args = lambda **k: (k.get("M", 8), 8, 8, A16, 16, A16, 16, k.get("lay", 1), k.get("sa", 1.0), 1.0,
                        A16, 8, 0, None)
    assert lib.tg_gemm_fp8(*args(M=-1)) == tg.TG_ERR_INVALID_VALUE
    assert lib.tg_gemm_fp8(*args(sa=float("inf"))) == tg.TG_ERR_INVALID_VALUE
    # row-major B: ldb >= N, and N bytes per row a multiple of 16
    assert lib.tg_gemm_fp8(8, 32, 8, A16, 16, A16, 16, 0, 1.0, 1.0, A16, 32, 0, None) == tg.TG_ERR_INVALID_VALUE
    assert lib.tg_gemm_fp8(8, 24, 8, A16, 16, A16, 24, 0, 1.0, 1.0, A16, 24, 0, None) == tg.TG_ERR_MISALIGNED
    assert lib.tg_gemm_fp8(*args(M=0)) == tg.TG_OK
    # fp8 rows of 8 elements are only 8 bytes: misaligned leading dimension
    assert lib.tg_gemm_fp8(8, 8, 8, A16, 8, A16, 16, 1, 1.0, 1.0, A16, 8, 0, None) == tg.TG_ERR_MISALIGNED


def test_w4a16_validation(tg):
    lib = tg.lib

    def call(M=4, N=8, K=128, A=A16, lda=128, q=A16, ldq=16, s=A16, lds=1, g=128, zp=8, C=A16, ldc=8):
        return lib.tg_gemm_w4a16(M, N, K, A, lda, q, ldq, s, lds, g, zp, C, ldc, None)

    assert call(M=-1) == tg.TG_ERR_INVALID_VALUE
    assert call(g=64) == tg.TG_ERR_NOT_SUPPORTED
    assert call(K=200) == tg.TG_ERR_NOT_SUPPORTED
    assert call(zp=16) == tg.TG_ERR_NOT_SUPPORTED
    assert call(q=None) == tg.TG_ERR_INVALID_VALUE
    assert call(ldq=8) == tg.TG_ERR_INVALID_VALUE
    assert call(lds=0) == tg.TG_ERR_INVALID_VALUE
    assert call(ldq=17) == tg.TG_ERR_MISALIGNED
    assert call(s=A16 + 1) == tg.TG_ERR_MISALIGNED
    assert call(A=A16 + 2) == tg.TG_ERR_MISALIGNED
    assert call(ldc=4) == tg.TG_ERR_INVALID_VALUE
    assert call(M=0) == tg.TG_OK
    assert lib.tg_dequant_w4(8, 128, A16, 16, A16, 1, 128, 8, None, 128, None) == tg.TG_ERR_INVALID_VALUE
    assert lib.tg_dequant_w4(8, 128, A16, 16, A16, 1, 128, 8, A16 + 2, 128, None) == tg.TG_ERR_MISALIGNED
    assert lib.tg_dequant_w4(8, 100, A16, 16, A16, 1, 128, 8, A16, 128, None) == tg.TG_ERR_NOT_SUPPORTED
    assert lib.tg_dequant_w4(0, 128, None, 16, None, 1, 128, 8, None, 128, None) == tg.TG_OK


def test_sp24_validation(tg):
    lib = ctypes.CDLL(tg.LIB_PATH)
    lib.tg_gemm_sp24_bf16.argtypes = [ctypes.c_int64] * 3 + [ctypes.c_void_p, ctypes.c_int64] * 4 + [ctypes.c_int,
                                                                                                    ctypes.c_void_p]
    P = 1 << 20  # a fake 1 MiB-aligned device address: validation never dereferences it

    def call(M=64, N=64, K=128, A=P, lda=128, V=P, ldv=64, W=P, ldm=16, C=P, ldc=64, dt=2):
        return lib.tg_gemm_sp24_bf16(M, N, K, A, lda, V, ldv, W, ldm, C, ldc, dt, None)

    assert call(M=-1) == tg.TG_ERR_INVALID_VALUE
    assert call(K=-64) == tg.TG_ERR_INVALID_VALUE
    assert call(dt=7) == tg.TG_ERR_INVALID_VALUE
    assert call(K=96) == tg.TG_ERR_NOT_SUPPORTED       # K not a multiple of 64
    assert call(M=0) == tg.TG_OK and call(N=0) == tg.TG_OK
    assert call(C=0) == tg.TG_ERR_INVALID_VALUE
    assert call(ldc=63) == tg.TG_ERR_INVALID_VALUE
    assert call(A=0) == tg.TG_ERR_INVALID_VALUE and call(V=0) == tg.TG_ERR_INVALID_VALUE
    assert call(W=0) == tg.TG_ERR_INVALID_VALUE
    assert call(lda=127) == tg.TG_ERR_INVALID_VALUE    # lda < K
    assert call(ldv=63) == tg.TG_ERR_INVALID_VALUE     # ldv < K/2
    assert call(ldm=15) == tg.TG_ERR_INVALID_VALUE     # ldm < K/8
    assert call(A=P + 2) == tg.TG_ERR_MISALIGNED
    assert call(V=P + 8) == tg.TG_ERR_MISALIGNED
    assert call(lda=132) == tg.TG_ERR_MISALIGNED       # lda*2 not a multiple of 16
    assert call(ldv=68) == tg.TG_ERR_MISALIGNED
    assert call(W=P + 2) == tg.TG_ERR_MISALIGNED       # codes need 4-byte alignment
    assert call(ldm=18) == tg.TG_ERR_MISALIGNED
    assert call(C=P + 4) == tg.TG_ERR_MISALIGNED
    assert call(ldc=66, dt=2) == tg.TG_ERR_MISALIGNED  # 66 bf16 = 132 bytes
    assert call(lda=1 << 30) == tg.TG_ERR_NOT_SUPPORTED  # offsets past the buffer-resource range


def test_product_and_oracle_share_no_code():
    """The oracle is independent of the HIP path: neither imports the other."""
    pkg = os.path.join(ROOT, "tile_level_gemm_02_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "oracle.c" not in text and "liboracle" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f), encoding="utf-8").read()
            assert not re.search(r"^\s*(import|from)\s+tile_level_gemm_02_amd\b", text, re.M), f
            assert not re.search(r"#\s*include\s*[<\"].*tg(_\w+)?\.h", text), f
            assert "libtg" not in text, f


def test_package_imports_without_the_library(tmp_path):
    """A checkout with no libtg.so built: the package and its build module
    import (so the library can be built from it), and the first entry-point
    call raises ImportError -- there is no fallback."""
    import shutil
    import subprocess
    import sys

    pkg = os.path.join(ROOT, "tile_level_gemm_02_amd")
    dst = tmp_path / "tile_level_gemm_02_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    assert not (dst / "libtg.so").exists()
    code = (
        "import tile_level_gemm_02_amd.build as b, tile_level_gemm_02_amd as t\n"
        "assert callable(b.build)\n"
        "try:\n"
        "    t.tg_version()\n"
        "except ImportError as e:\n"
        "    print('raised', 'not built' in str(e))\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "raised True", r.stdout


def test_gemm_ex_validation(tg):
    """tg_gemm_ex rejects bad workspace arguments before any HIP call."""
    lib = tg.lib
    W = 1 << 20  # a fake 256-byte aligned device address: validation never dereferences it

    def call(inp=1, M=256, N=8192, K=8192, lda=8192, ldb=8192, ws=W, nbytes=1 << 30, lay=1):
        return lib.tg_gemm_ex(inp, M, N, K, W, lda, W, ldb, lay, 1.0, 1.0, W, N, 2, ws, nbytes, None)

    need = lib.tg_gemm_ex_workspace_bytes(1, 256, 8192, 8192, 1)
    assert need > 65536
    assert lib.tg_gemm_ex_workspace_bytes(1, -1, 8, 8, 1) == -1
    assert lib.tg_gemm_ex_workspace_bytes(7, 8, 8, 8, 1) == -1
    assert lib.tg_gemm_ex_workspace_bytes(1, 4096, 4096, 4096, 1) == 0  # enough tiles: no split
    assert call(inp=5) == tg.TG_ERR_INVALID_VALUE
    assert call(nbytes=-1) == tg.TG_ERR_INVALID_VALUE
    assert call(ws=None, nbytes=256) == tg.TG_ERR_INVALID_VALUE
    assert call(nbytes=need - 1) == tg.TG_ERR_INVALID_VALUE  # smaller than the query reports
    assert call(ws=W + 16) == tg.TG_ERR_MISALIGNED          # not 256-byte aligned
    assert call(M=-1) == tg.TG_ERR_INVALID_VALUE
    assert call(M=0) == tg.TG_OK and call(N=0) == tg.TG_OK
    assert call(lda=8) == tg.TG_ERR_INVALID_VALUE            # the dense checks still apply


def test_gemm_ex_noalloc_validation(tg):
    """tg_gemm_ex_noalloc checks every argument before its first HIP call."""
    lib = tg.lib
    W = 1 << 20

    def call(inp=1, M=256, N=8192, K=8192, lda=8192, C=W, cd=2, sa=1.0):
        return lib.tg_gemm_ex_noalloc(inp, M, N, K, W, lda, W, K, 1, sa, 1.0, C, N, cd, None)

    assert call(inp=9) == tg.TG_ERR_INVALID_VALUE
    assert call(M=-1) == tg.TG_ERR_INVALID_VALUE
    assert call(lda=8) == tg.TG_ERR_INVALID_VALUE
    assert call(C=None) == tg.TG_ERR_INVALID_VALUE
    assert call(C=W + 2) == tg.TG_ERR_MISALIGNED
    assert call(cd=7) == tg.TG_ERR_INVALID_VALUE
    assert call(inp=2, sa=float("nan")) == tg.TG_ERR_INVALID_VALUE
    assert call(M=0) == tg.TG_OK
    assert "static buffer" in tg.tg_status_string(tg.TG_ERR_SCRATCH)


def test_w4a16_ex_validation(tg):
    lib = tg.lib
    W = 1 << 20

    def call(M=256, N=8192, K=8192, ws=W, nbytes=1 << 30, g=128):
        return lib.tg_gemm_w4a16_ex(M, N, K, W, K, W, K // 8, W, K // 128, g, 8, W, N, ws, nbytes, None)

    need = lib.tg_gemm_w4a16_ex_workspace_bytes(256, 8192, 8192)
    assert need > 65536
    assert lib.tg_gemm_w4a16_ex_workspace_bytes(16, 8192, 8192) == 0  # decode sizes: no split
    assert lib.tg_gemm_w4a16_ex_workspace_bytes(-1, 8, 128) == -1
    assert call(nbytes=-1) == tg.TG_ERR_INVALID_VALUE
    assert call(ws=None, nbytes=256) == tg.TG_ERR_INVALID_VALUE
    assert call(nbytes=need - 1) == tg.TG_ERR_INVALID_VALUE
    assert call(ws=W + 64) == tg.TG_ERR_MISALIGNED
    assert call(g=64) == tg.TG_ERR_NOT_SUPPORTED  # the w4a16 checks still apply
    assert call(M=0) == tg.TG_OK
