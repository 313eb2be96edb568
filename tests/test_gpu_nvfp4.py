"""GPU parity of the W4A16 NVFP4 calls (dequantisation, GEMV, tiled GEMM)."""

import numpy as np
import pytest
import torch

import synth
from oracle import compare as C
from oracle import formats as F
from oracle import ref as R
from gpu_util import bf16_bits, show, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import weight_quantized_linear_amd as q
    return q


def test_dequant_every_byte_and_scale_bit_exact(q):
    """Rows hold all 256 packed bytes (every nibble pair, both nibble
    positions); each row uses a different block scale, over all 254 finite
    E4M3 codes (subnormal, zero, 448, negative)."""
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    n, k = len(finite), 512
    packed = np.tile(np.arange(256, dtype=np.uint8), (n, 1))
    scales = np.repeat(finite[:, None], k // 16, axis=1)
    want = R.nvfp4_dequant(packed, scales)
    p, s = to_dev_u8(packed), to_dev_u8(scales)
    show("nvfp4 dequant bf16")
    got = bf16_bits(q.nvfp4_dequant(p, s, torch.bfloat16))
    assert np.array_equal(got, F.f64_to_bf16_bits(want))
    show("nvfp4 dequant f32")
    gf = q.nvfp4_dequant(p, s, torch.float32).cpu().numpy()
    assert np.array_equal(gf.view(np.uint32), want.astype(np.float32).view(np.uint32))


def test_identity_activation_gives_transposed_dequant(q):
    """X = I_K through the tiled path: out = D^T, one exact product per output."""
    k = 256
    packed, scales, _ = synth.nvfp4_weight((50,), 300, k)
    eye = synth.bf16_bits_from_f32(np.eye(k, dtype=np.float32))
    show("nvfp4 identity")
    out = q.nvfp4_gemm(to_dev_u8(packed), to_dev_u8(scales), to_dev_bf16(eye), out_dtype=torch.float32, path="tiled")
    assert np.array_equal(out.cpu().numpy().astype(np.float64), R.nvfp4_dequant(packed, scales).T)


def test_gemv_one_hot_returns_dequantised_column(q):
    packed, scales, _ = synth.nvfp4_weight((51,), 333, 4096)
    d = R.nvfp4_dequant(packed, scales)
    p, s = to_dev_u8(packed), to_dev_u8(scales)
    for kk in (0, 1, 15, 16, 4095):
        x = np.zeros((1, 4096), np.uint16)
        x[0, kk] = 0x3F80
        show("nvfp4 one-hot", kk)
        out = q.nvfp4_gemm(p, s, to_dev_bf16(x), out_dtype=torch.float32, path="gemv")
        assert np.array_equal(out.cpu().numpy()[0].astype(np.float64), d[:, kk])


NVFP4_DYADIC = [("gemv", 1, 7, 4096), ("gemv", 1, 515, 48), ("gemv", 3, 129, 2048), ("gemv", 4, 1000, 4096),
                ("gemv", 2, 65, 4112), ("tiled", 5, 100, 4096), ("tiled", 128, 300, 1024),
                ("tiled", 200, 129, 2064), ("tiled", 1, 17, 16),
                # 128x256 tiles (ragged N; strips of 64 values, K % 128 == 64, and of 128 values: one and
                # three) and 256x256 tiles (ragged M)
                ("tiled", 2048, 2100, 64), ("tiled", 2048, 2100, 192), ("tiled", 2048, 4096, 128),
                ("tiled", 2048, 2100, 384), ("tiled", 4100, 4096, 64),
                # split-K: 64-row tiles up to M = 256 (the M = 128 workload shape), 128-row above
                ("tiled", 128, 4096, 4096), ("tiled", 77, 1000, 2048), ("tiled", 256, 640, 1024),
                ("tiled", 257, 640, 1024),
                # split-K with nine 128-value strips over three slices, and seventeen 64-value strips
                ("tiled", 128, 4096, 1152), ("tiled", 100, 2048, 1088),
                # 128x128 tiles of four side-by-side waves with 64-value strips (at most half of the
                # CUs would get a 128x256 tile): exactly half, and ragged M and N with five and
                # sixty-five strips
                ("tiled", 1024, 4096, 256), ("tiled", 1000, 1030, 320), ("tiled", 640, 770, 4160)]


@pytest.mark.parametrize("path,m,n,k", NVFP4_DYADIC)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dyadic_bit_exact(q, path, m, n, k, out_dtype):
    packed, scales = synth.dyadic_nvfp4_weight((52, m, n, k), n, k)
    x = synth.dyadic_activation((53, m, n, k), m, k)
    ref, _ = R.nvfp4_linear(packed, scales, x)
    show("nvfp4 dyadic", path, m, n, k, out_dtype)
    out = q.nvfp4_gemm(to_dev_u8(packed), to_dev_u8(scales), to_dev_bf16(x), out_dtype=out_dtype, path=path)
    if out_dtype == torch.float32:
        assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))
    else:
        assert np.array_equal(bf16_bits(out), F.f64_to_bf16_bits(ref))


@pytest.fixture(scope="module")
def nvfp4_weight():
    return synth.nvfp4_weight((3, 0, 0), 4096, 4096)


@pytest.mark.parametrize("m", [1, 128, 2048])
def test_nvfp4_workload_bf16(q, nvfp4_weight, m):
    c = synth.config3_case(m, weight=nvfp4_weight)
    ref, bound = R.nvfp4_linear(c.w_packed, c.w_scale, c.x, c.alpha)
    show("nvfp4 workload", c.name)
    out = q.nvfp4_gemm(to_dev_u8(c.w_packed), to_dev_u8(c.w_scale), to_dev_bf16(c.x), alpha=c.alpha)
    res = C.check_bf16(bf16_bits(out), ref, C.fp_tolerance(bound))
    assert res and res.n_clause2 <= C.clause2_budget(ref), res


def test_nvfp4_workload_f32_m128(q, nvfp4_weight):
    c = synth.config3_case(128, weight=nvfp4_weight)
    ref, bound = R.nvfp4_linear(c.w_packed, c.w_scale, c.x, c.alpha)
    show("nvfp4 f32")
    out = q.nvfp4_gemm(to_dev_u8(c.w_packed), to_dev_u8(c.w_scale), to_dev_bf16(c.x), alpha=c.alpha,
                       out_dtype=torch.float32)
    res = C.check_f32(out.cpu().numpy(), ref, bound)
    assert res and res.max_rel < 1e-5, res


def test_gemv_and_tiled_agree_on_exact_inputs(q):
    packed, scales = synth.dyadic_nvfp4_weight((54,), 640, 2048)
    x = synth.dyadic_activation((55,), 4, 2048)
    args = (to_dev_u8(packed), to_dev_u8(scales), to_dev_bf16(x))
    show("nvfp4 cross-path")
    a = q.nvfp4_gemm(*args, out_dtype=torch.float32, path="gemv")
    b = q.nvfp4_gemm(*args, out_dtype=torch.float32, path="tiled")
    assert torch.equal(a, b)


def test_nvfp4_rejects_k_not_multiple_of_16(q):
    p = torch.zeros((4, 12), dtype=torch.uint8, device="cuda:0")
    s = torch.zeros((4, 2), dtype=torch.uint8, device="cuda:0")
    x = torch.zeros((1, 24), dtype=torch.bfloat16, device="cuda:0")
    st = q.lib.qlinear_nvfp4_gemm(p.data_ptr(), s.data_ptr(), x.data_ptr(), x.data_ptr(), 0, 1, 4, 24, 1.0, None)
    assert st == q.ERR_INVALID_ARG
