"""GPU parity of the dense bf16 control (qlinear_bf16_gemm: GEMV, skinny and
tiled kernel families) against the CPU oracle, through the C ABI."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import compare as C
from oracle import formats as F
from oracle import ref as R
from gpu_util import bf16_bits, show, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import weight_quantized_linear_amd as q
    return q


# ------------------------------------------------------------------ exact (dyadic) inputs

DYADIC = [
    # vector-ALU GEMV: wide loads (K % 8 == 0) and the element-wise kernel
    ("gemv", 1, 1, 8), ("gemv", 1, 7, 4096), ("gemv", 1, 515, 2050), ("gemv", 1, 33, 3),
    ("gemv", 1, 4100, 8192), ("gemv", 2, 129, 2064), ("gemv", 3, 5, 48), ("gemv", 4, 1031, 4096),
    ("gemv", 4, 70, 2050),
    # 16x16x32 skinny kernel: one and four 16-column groups per block, ragged N, K not a multiple of 32
    ("skinny", 1, 17, 8), ("skinny", 5, 33, 4104), ("skinny", 16, 1000, 1040), ("skinny", 16, 8200, 4096),
    ("skinny", 11, 2000, 14336), ("skinny", 4, 9000, 520),
    # tiled: split-K (small M), 128x128 and 256x128 LDS tiles with ragged edges, the register-staged
    # kernel for K % 64 != 0 and for K % 8 != 0
    ("tiled", 1, 300, 4096), ("tiled", 17, 1000, 1024), ("tiled", 300, 520, 2048),
    ("tiled", 1030, 8200, 128), ("tiled", 40, 72, 1000), ("tiled", 33, 130, 1001),
    ("auto", 16, 4096, 4096), ("auto", 64, 2048, 2048), ("auto", 3, 100, 5),
]


@pytest.mark.parametrize("path,m,n,k", DYADIC)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dyadic_inputs_are_bit_exact(q, path, m, n, k, out_dtype):
    wb = synth.dyadic_bf16_weight((30, m, n, k), n, k)
    xb = synth.dyadic_activation((31, m, n, k), m, k)
    ref, _ = R.bf16_linear(wb, xb)
    show("bf16 dyadic", path, m, n, k, out_dtype)
    out = q.bf16_gemm(to_dev_bf16(wb), to_dev_bf16(xb), out_dtype=out_dtype, path=path)
    if out_dtype == torch.float32:
        assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))
    else:
        assert np.array_equal(bf16_bits(out), F.f64_to_bf16_bits(ref))


# ------------------------------------------------------------------ random inputs, every family

@pytest.mark.parametrize("path,m,n,k", [
    ("gemv", 1, 2048, 2048), ("gemv", 4, 333, 4096), ("gemv", 2, 99, 1001),
    ("skinny", 7, 1500, 4096), ("skinny", 16, 9000, 2048),
    ("tiled", 1, 2048, 4096), ("tiled", 200, 700, 2048), ("tiled", 1024, 8192, 256), ("tiled", 50, 90, 1000),
])
def test_random_inputs_within_tolerance(q, path, m, n, k):
    wb = synth.bf16_weight((32, m, n, k), n, k)
    xb = synth.bf16_activation((33, m, n, k), m, k)
    ref, bound = R.bf16_linear(wb, xb, 0.75)
    w, x = to_dev_bf16(wb), to_dev_bf16(xb)
    show("bf16 random f32", path, m, n, k)
    got = q.bf16_gemm(w, x, out_dtype=torch.float32, alpha=0.75, path=path).cpu().numpy()
    res = C.check_f32(got, ref, bound)
    assert res, res
    show("bf16 random bf16", path, m, n, k)
    gb = bf16_bits(q.bf16_gemm(w, x, out_dtype=torch.bfloat16, alpha=0.75, path=path))
    res = C.check_bf16(gb, ref, C.fp_tolerance(bound))
    assert res, res
    assert res.n_clause2 <= C.clause2_budget(ref), res


# ------------------------------------------------------------------ the decode shapes with bf16 weights

@pytest.fixture(scope="module")
def decode_weights():
    cache = {}

    def get(idx):
        if idx not in cache:
            n, k = synth.CONFIG2_SHAPES[idx]
            wb = synth.bf16_weight((34, idx), n, k)
            cache.clear()  # keep one weight resident at a time
            cache[idx] = (wb, to_dev_bf16(wb))
        return cache[idx]
    return get


@pytest.mark.parametrize("shape_idx", [0, 1, 2, 3])
@pytest.mark.parametrize("m", synth.CONFIG2_M)
def test_decode_shapes(q, decode_weights, shape_idx, m):
    wb, w = decode_weights(shape_idx)
    n, k = wb.shape
    xb = synth.bf16_activation((35, shape_idx, m), m, k)
    show("bf16 decode shape", m, n, k)
    got = bf16_bits(q.bf16_gemm(w, to_dev_bf16(xb), out_dtype=torch.bfloat16))
    if n > 20000:  # rows the oracle computes one by one, plus both ends
        rows = np.unique(np.concatenate([np.random.default_rng(shape_idx).choice(n, 3000, replace=False),
                                         np.arange(n - 70, n), np.arange(0, 64)]))
    else:
        rows = np.arange(n)
    ref, bound = R.bf16_linear(wb[rows], xb)
    res = C.check_bf16(got[:, rows], ref, C.fp_tolerance(bound))
    assert res, res
    assert res.n_clause2 <= C.clause2_budget(ref), res


# ------------------------------------------------------------------ hygiene and errors

@pytest.mark.parametrize("path,m", [("gemv", 2), ("skinny", 9), ("tiled", 40)])
def test_writes_stay_inside_out(q, path, m):
    n, k = 333, 1024
    wb = synth.bf16_weight((36, m), n, k)
    xb = synth.bf16_activation((37, m), m, k)
    buf = torch.full((m * n + 4096,), float("nan"), dtype=torch.float32, device="cuda:0")
    show("bf16 stray", path, m)
    q.bf16_gemm(to_dev_bf16(wb), to_dev_bf16(xb), out=buf[: m * n].view(m, n), out_dtype=torch.float32, path=path)
    assert np.all(np.isnan(buf[m * n:].cpu().numpy()))
    assert not np.any(np.isnan(buf[: m * n].cpu().numpy()))


def test_c_abi_rejects_bad_arguments(q):
    lib = q.lib
    w = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda:0")
    x = torch.zeros((20, 128), dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty((20, 64), dtype=torch.float32, device="cuda:0")
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    odd = ctypes.c_void_p(w.data_ptr() + 1)
    show("bf16 bad args")
    assert lib.qlinear_bf16_gemm(p(w), p(x), p(out), 0, 20, 64, 128, 1.0, None) == 0
    assert lib.qlinear_bf16_gemm(odd, p(x), p(out), 0, 20, 64, 128, 1.0, None) == q.ERR_INVALID_ARG
    assert lib.qlinear_bf16_gemm(p(w), p(x), p(out), 0, 0, 64, 128, 1.0, None) == q.ERR_INVALID_ARG
    assert lib.qlinear_bf16_gemm(p(w), p(x), p(out), 2, 20, 64, 128, 1.0, None) == q.ERR_INVALID_ARG
    assert lib.qlinear_bf16_gemm_path(p(w), p(x), p(out), 0, 20, 64, 128, 1.0, 1, None) == q.ERR_INVALID_ARG
    assert lib.qlinear_bf16_gemm_path(p(w), p(x), p(out), 0, 17, 64, 128, 1.0, 2, None) == q.ERR_INVALID_ARG
    assert lib.qlinear_bf16_gemm_path(p(w), p(x), p(out), 0, 20, 64, 128, 1.0, 9, None) == q.ERR_INVALID_ARG
    torch.cuda.synchronize()
