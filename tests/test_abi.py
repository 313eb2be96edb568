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
    assert q.lib.qlinear_abi_version() == 1
    assert q.lib.qlinear_status_string(0) == b"ok"
    for s in range(1, 5):
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
