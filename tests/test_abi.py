"""The C-ABI library loads and exports every symbol include/qlinear.h
declares; argument validation answers before any device work (CPU only)."""

import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qlinear.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(qlinear_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def q():
    import weight_quantized_linear_amd as q
    return q


def test_header_declares_the_calls():
    names = declared_functions()
    for must in ("qlinear_fp8_gemv", "qlinear_fp8_gemm", "qlinear_fp8_materialize", "qlinear_abi_version"):
        assert must in names


def test_library_exports_every_declared_symbol(q):
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(qlinear_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    # the binding knows every declared call, and nothing else
    assert set(q.EXPORTED) == set(names)
    for n in names:
        assert getattr(q.lib, n) is not None


def test_version_and_status_strings(q):
    assert q.lib.qlinear_abi_version() == 2
    assert q.lib.qlinear_status_string(0) == b"ok"
    for s in range(1, 6):
        assert q.lib.qlinear_status_string(s) not in (b"ok", b"unknown status")
    assert q.lib.qlinear_status_string(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args", [
    (None, FAKE, FAKE, 0, 8, 16, 1.0),        # null weight
    (FAKE, None, FAKE, 0, 8, 16, 1.0),        # null x
    (FAKE, FAKE, None, 0, 8, 16, 1.0),        # null out
    (FAKE, FAKE, FAKE, 0, 0, 16, 1.0),        # N = 0
    (FAKE, FAKE, FAKE, 0, 8, -1, 1.0),        # K < 0
    (FAKE, FAKE, FAKE, 2, 8, 16, 1.0),        # I32 output not allowed
    (FAKE, FAKE, FAKE, 7, 8, 16, 1.0),        # unknown dtype
    (FAKE, FAKE, FAKE, 0, 1 << 40, 1 << 40, 1.0),  # N*K overflows
])
def test_gemv_rejects_bad_arguments(q, args):
    assert q.lib.qlinear_fp8_gemv(*args, None) == q.ERR_INVALID_ARG


def test_gemm_rejects_bad_arguments(q):
    L = q.lib
    assert L.qlinear_fp8_gemm(FAKE, FAKE, FAKE, 0, 0, 8, 16, 1.0, None) == q.ERR_INVALID_ARG
    assert L.qlinear_fp8_gemm(FAKE, FAKE, ctypes.c_void_p(0x10001), 0, 1, 8, 16, 1.0, None) == q.ERR_INVALID_ARG
    # forced families that cannot take the shape
    assert L.qlinear_fp8_gemm_path(FAKE, FAKE, FAKE, 0, 5, 8, 16, 1.0, 1, None) == q.ERR_INVALID_ARG
    assert L.qlinear_fp8_gemm_path(FAKE, FAKE, FAKE, 0, 17, 8, 16, 1.0, 2, None) == q.ERR_INVALID_ARG
    assert L.qlinear_fp8_gemm_path(FAKE, FAKE, FAKE, 0, 4, 8, 17, 1.0, 2, None) == q.ERR_INVALID_ARG
    assert L.qlinear_fp8_gemm_path(FAKE, FAKE, FAKE, 0, 4, 8, 16, 1.0, 9, None) == q.ERR_INVALID_ARG
    assert L.qlinear_fp8_materialize(FAKE, None, 0, 4, 4, None) == q.ERR_INVALID_ARG
    assert L.qlinear_fp8_materialize(FAKE, FAKE, 2, 4, 4, None) == q.ERR_INVALID_ARG


def test_workspace_arguments_rejected_before_device_work(q):
    """The caller-owned split-K workspace: a misaligned one, a negative size or
    a NULL one with a size are argument errors, answered before any device
    query; so are bad arguments of the size query."""
    L = q.lib
    ws_bad = [(ctypes.c_void_p(0x10008), 1024), (FAKE, -1), (None, 64)]
    for ws, nb in ws_bad:
        assert L.qlinear_fp8_gemm_ws(FAKE, FAKE, FAKE, 0, 32, 64, 64, 1.0, None, 0, ws, nb, None) == q.ERR_INVALID_ARG
        assert L.qlinear_bf16_gemm_ws(FAKE, FAKE, FAKE, 0, 32, 64, 64, 1.0, None, 0, ws, nb, None) == \
            q.ERR_INVALID_ARG
        assert L.qlinear_nvfp4_gemm_ws(FAKE, FAKE, FAKE, FAKE, 0, 32, 64, 64, 1.0, None, 0, ws, nb, None) == \
            q.ERR_INVALID_ARG
    b = ctypes.c_int64(-5)
    assert L.qlinear_gemm_workspace_size(0, 0, 16, 64, 64, None) == q.ERR_INVALID_ARG
    assert L.qlinear_gemm_workspace_size(3, 0, 16, 64, 64, ctypes.byref(b)) == q.ERR_INVALID_ARG  # format
    assert b.value == 0
    assert L.qlinear_gemm_workspace_size(0, 5, 16, 64, 64, ctypes.byref(b)) == q.ERR_INVALID_ARG  # path
    assert L.qlinear_gemm_workspace_size(1, 0, 16, 64, 40, ctypes.byref(b)) == q.ERR_INVALID_ARG  # NVFP4 K % 16
    assert L.qlinear_gemm_workspace_size(0, 0, 0, 64, 64, ctypes.byref(b)) == q.ERR_INVALID_ARG  # M = 0


C_CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "qlinear.h"
int main(void) {
  if (qlinear_abi_version() != QLINEAR_ABI_VERSION) return 1;
  if (strcmp(qlinear_status_string(QLINEAR_OK), "ok") != 0) return 2;
  if (qlinear_fp8_gemv(NULL, NULL, NULL, QLINEAR_F32, 8, 16, 1.0f, NULL) != QLINEAR_ERR_INVALID_ARG) return 3;
  if (qlinear_int8_quantize_act(NULL, NULL, NULL, 4, 4, NULL) != QLINEAR_ERR_INVALID_ARG) return 4;
  if (qlinear_gemm_workspace_size(QLINEAR_WEIGHT_FP8, QLINEAR_PATH_AUTO, 16, 64, 64, NULL) != QLINEAR_ERR_INVALID_ARG)
    return 5;
  puts("c client ok");
  return 0;
}
"""


@pytest.mark.skipif(subprocess.run(["which", "gcc"], capture_output=True).returncode != 0, reason="no gcc")
def test_plain_c_client_compiles_links_and_runs(q, tmp_path):
    """The header is plain C99 (and valid C++17); a C program links against
    the library and calls it (no device work: version, status text, argument
    rejection)."""
    inc = os.path.join(ROOT, "include")
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    libdir = os.path.dirname(q.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{inc}", str(src),
                    f"-L{libdir}", "-lqlinear", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True)
    assert run.returncode == 0 and run.stdout.strip() == "c client ok", (run.returncode, run.stdout, run.stderr)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", "-x", "c++",
                    HEADER], check=True)
