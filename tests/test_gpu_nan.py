"""NaN codes through every kernel family (the degenerate input the formats
have: E4M3 0x7F / 0xFF decode to NaN, an E4M3 block scale likewise).  A NaN
weight byte must make exactly its output column NaN, for every activation
row (0 x NaN is NaN), and leave every other output bit-exact; a NaN
activation code in W8A8 makes exactly its output row NaN.  Inputs are dyadic,
so the finite outputs must equal the oracle's bit for bit."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import ref as R
from gpu_util import DEV, bf16_bits, show, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import weight_quantized_linear_amd as q
    return q


def _check(out, ref, out_dtype):
    nan = np.isnan(ref)
    if out_dtype == torch.float32:
        got = out.cpu().numpy()
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].astype(np.float32).view(np.uint32))
    else:
        gb = bf16_bits(out)
        assert np.array_equal((gb & 0x7FFF) > 0x7F80, nan)
        assert np.array_equal(gb[~nan], F.f64_to_bf16_bits(ref[~nan]))


def _plant(codes, r, count=3):
    """NaN codes at `count` random (n, k) places, both signs; returns their columns."""
    n, k = codes.shape
    cols = r.choice(n, size=min(count, n), replace=False)
    for i, c in enumerate(cols):
        codes[c, r.integers(0, k)] = 0x7F if i % 2 == 0 else 0xFF
    return cols


FP8_CASES = [("gemv", 1, 300, 4096), ("gemv", 3, 300, 2050), ("gemv", 2, 4100, 1000),
             ("skinny", 4, 70000, 256), ("skinny", 16, 65601, 528), ("skinny", 8, 300, 4096),
             ("skinny", 3, 200, 1008), ("splitk", 16, 1000, 8192), ("tiled", 300, 700, 1024),
             ("tiled", 100, 300, 1000), ("auto", 2048, 512, 512)]


@pytest.mark.parametrize("path,m,n,k", FP8_CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fp8_nan_weight_poisons_its_column_only(q, path, m, n, k, out_dtype):
    r = np.random.default_rng([m, n, k])
    wc = synth.dyadic_fp8_weight((90, m, n, k), n, k)
    cols = _plant(wc, r)
    xc = synth.dyadic_activation((91, m, n, k), m, k)
    ref, _ = R.fp8_linear(wc, xc)
    assert np.all(np.isnan(ref[:, cols])) and np.isnan(ref).sum() == m * len(cols)
    show("nan fp8", path, m, n, k, out_dtype)
    out = q.fp8_gemm(to_dev_u8(wc), to_dev_bf16(xc), out_dtype=out_dtype, path=path)
    _check(out, ref, out_dtype)


@pytest.mark.parametrize("path,m,n,k", [("gemv", 1, 300, 4096), ("gemv", 4, 129, 2048), ("tiled", 128, 640, 1024),
                                        ("tiled", 2048, 512, 256), ("tiled", 77, 300, 2064)])
def test_nvfp4_nan_block_scale_poisons_its_column_only(q, path, m, n, k):
    r = np.random.default_rng([m, n, k, 4])
    packed, scales = synth.dyadic_nvfp4_weight((92, m, n, k), n, k)
    cols = _plant(scales, r)
    x = synth.dyadic_activation((93, m, n, k), m, k)
    ref, _ = R.nvfp4_linear(packed, scales, x)
    assert np.all(np.isnan(ref[:, cols])) and np.isnan(ref).sum() == m * len(cols)
    show("nan nvfp4", path, m, n, k)
    out = q.nvfp4_gemm(to_dev_u8(packed), to_dev_u8(scales), to_dev_bf16(x), out_dtype=torch.float32, path=path)
    _check(out, ref, torch.float32)


@pytest.mark.parametrize("m,n,k", [(300, 700, 1024), (2048, 512, 512), (33, 17, 2050)])
def test_fp8_w8a8_nan_codes_poison_their_row_and_column(q, m, n, k):
    r = np.random.default_rng([m, n, k, 8])
    xq = synth.dyadic_e4m3_activation((94, m, n, k), m, k)
    w = synth.dyadic_fp8_weight((95, m, n, k), n, k)
    cols = _plant(w, r, 2)
    rows = _plant(xq, r, 2)
    ref, _ = R.fp8_w8a8_linear(xq, w, 0.5)
    assert np.all(np.isnan(ref[rows, :])) and np.all(np.isnan(ref[:, cols]))
    show("nan w8a8", m, n, k)
    out = q.fp8_w8a8_gemm(to_dev_u8(xq), to_dev_u8(w), out_dtype=torch.float32, alpha=0.5)
    _check(out, ref, torch.float32)


def test_grouped_nan_weight_poisons_its_column_in_that_experts_rows(q):
    e, n, k, t = 4, 200, 1024, 300
    r = np.random.default_rng(96)
    w = synth.dyadic_fp8_weight((96,), e * n, k).reshape(e, n, k)
    col = 17
    w[2, col, 5] = 0x7F  # expert 2 only
    x = synth.dyadic_activation((97,), t, k)
    offs = np.array([0, 50, 120, 120, 260, 300])
    ids = np.array([2, 0, 3, 2, -1], np.int32)
    ref, _, written = R.fp8_grouped(w, x, offs, ids)
    nan = np.isnan(ref)
    expert2 = np.zeros(t, bool)
    expert2[0:50] = expert2[120:260] = True
    assert np.array_equal(nan.any(axis=1), expert2) and np.array_equal(np.flatnonzero(nan.any(axis=0)), [col])
    show("nan grouped")
    out = torch.full((t, n), 7.0, dtype=torch.float32, device=DEV)
    q.fp8_grouped_gemm(to_dev_u8(w), to_dev_bf16(x), torch.from_numpy(offs.astype(np.int32)).to(DEV),
                       torch.from_numpy(ids).to(DEV), out=out, out_dtype=torch.float32)
    assert written.all()
    _check(out, ref, torch.float32)
