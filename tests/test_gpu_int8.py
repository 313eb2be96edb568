"""GPU parity of the W8A8 int8 calls: activation quantiser (bit-exact codes
and scales) and int8 GEMM (bit-exact int32 accumulators; dequantised bf16)."""

import numpy as np
import pytest
import torch

import synth
from oracle import compare as C
from oracle import formats as F
from oracle import ref as R
from gpu_util import DEV, bf16_bits, show, to_dev_bf16, to_dev_i8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import weight_quantized_linear_amd as q
    return q


@pytest.fixture(scope="module")
def case3072():
    return synth.config5_case(3072)


def test_quantizer_workload_bit_exact(q, case3072):
    c = case3072
    show("int8 quantize", c.name)
    qd, sd = q.int8_quantize_act(to_dev_bf16(c.x))
    want_q, want_s = R.int8_quantize_act(c.x)
    assert np.array_equal(sd.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(qd.cpu().numpy(), want_q)


@pytest.mark.parametrize("m,k", [(5, 8), (7, 5000), (9, 4096), (3, 3), (6, 1001), (2, 8192 + 8)])
def test_quantizer_shapes_bit_exact(q, m, k):
    x = synth.bf16_activation((60, m, k), m, k, outlier_p=0.05)
    x[0, :] = 0                                             # zero row
    if m > 1:                                               # a row with exact ties: absmax 127 -> scale 1
        vals = np.resize(np.array([127.0, 2.5, -2.5, 3.5, -0.5, 0.5, -126.5, 1.5]), k)
        x[1] = F.f64_to_bf16_bits(vals)
    show("int8 quantize", m, k)
    qd, sd = q.int8_quantize_act(to_dev_bf16(x))
    want_q, want_s = R.int8_quantize_act(x)
    assert np.array_equal(sd.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(qd.cpu().numpy(), want_q)


def test_quantizer_quotients_near_half_integers(q):
    """Rows whose quotients x / scale fall on or next to half-integers (the
    kernel multiplies by 1 / scale and lets the IEEE division decide near a
    rounding boundary), plus a row whose scale is subnormal (division only)."""
    targets = [1.0 / 3.0, 0.7, 1e-3 * np.pi, 5.5e-30, 2.3e-5]
    n = np.arange(-126, 127, dtype=np.float64)
    rows = []
    for s_t in targets:
        vals = [127.0 * s_t]
        for eps in (0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -14, -(2.0 ** -14), 2.0 ** -7):
            vals.extend((n + 0.5 + eps) * s_t)
        rows.append(np.array(vals))
    k = max(len(r) for r in rows)
    x = np.zeros((len(rows) + 1, k), np.uint16)
    for i, r in enumerate(rows):
        x[i, :len(r)] = F.f64_to_bf16_bits(r)
    x[-1, :4] = [0x0001, 0x8003, 0x0007, 0x0000]  # bf16 subnormals: the scale is subnormal too
    want_q, want_s = R.int8_quantize_act(x)
    # the boundary cases are really there: fp32 quotients within 2^-14 of a half-integer
    xf = F.bf16_bits_to_f64(x[:-1]).astype(np.float32)
    ratio = np.divide(xf, want_s[:-1, None], dtype=np.float32)
    near = np.abs(np.abs(ratio - np.rint(ratio)) - 0.5) < 2.0 ** -14
    assert near.sum() >= 30
    assert want_s[-1] < np.float32(2.0 ** -126) and want_s[-1] > 0
    show("int8 quantize near halves")
    qd, sd = q.int8_quantize_act(to_dev_bf16(x))
    assert np.array_equal(sd.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(qd.cpu().numpy(), want_q)


def test_quantizer_non_finite_rows(q):
    """Rows holding a NaN, +inf or -inf (the reading of the oracle): a_scale
    NaN / +inf and zero codes, on the vector kernel and on the element-wise
    kernel (unaligned view); finite rows stay bit-exact."""
    m, k = 8, 1024
    x = synth.bf16_activation((62,), m, k + 1, outlier_p=0.01)
    nan, pinf, ninf = 0x7FC0, 0x7F80, 0xFF80
    x[1, 17] = nan
    x[2, 500] = pinf
    x[3, 3] = ninf
    x[4, 0], x[4, 900] = pinf, nan
    x[5, 1000] = 0xFFC1                                   # a negative NaN with a payload
    for name, xd, xs in (("vector", to_dev_bf16(np.ascontiguousarray(x[:, :k])), x[:, :k]),
                         ("element-wise", to_dev_bf16(x.reshape(-1))[1:1 + m * k].reshape(m, k),
                          x.reshape(-1)[1:1 + m * k].reshape(m, k))):
        show("int8 quantize non-finite", name)
        qd, sd = q.int8_quantize_act(xd)
        want_q, want_s = R.int8_quantize_act(xs)
        got_s = sd.cpu().numpy()
        assert np.array_equal(np.isnan(got_s), np.isnan(want_s)), name
        fin = ~np.isnan(want_s)
        assert np.array_equal(got_s[fin].view(np.uint32), want_s[fin].view(np.uint32)), name
        assert np.array_equal(qd.cpu().numpy(), want_q), name
        assert np.sum(~np.isfinite(want_s)) >= 4


def test_quantizer_unaligned_view(q):
    x = synth.bf16_activation((61,), 1, 4 * 1000 + 1)
    xd = to_dev_bf16(x)[0, 1:].reshape(4, 1000)            # base not 16-byte aligned
    show("int8 quantize unaligned")
    qd, sd = q.int8_quantize_act(xd)
    want_q, want_s = R.int8_quantize_act(x[0, 1:].reshape(4, 1000))
    assert np.array_equal(qd.cpu().numpy(), want_q) and np.array_equal(sd.cpu().numpy(), want_s)


# (4000, 3000, 1024): 256 x 256 tiles with 128-byte strips, ragged in both directions;
# (4000, 3000, 1088) the same tiles with 64-byte strips (K % 128 == 64); (2048, 4096, 128 / 256)
# one and two 128-byte strips (a ring of two stages, the prologue re-fetching the last strip)
@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (130, 70, 100), (257, 129, 4099), (128, 256, 3072), (333, 1000, 64),
                                   (4000, 3000, 1024), (4000, 3000, 1088), (2048, 4096, 128), (2048, 4096, 256)])
def test_int32_accumulators_bit_exact(q, m, n, k):
    r = np.random.default_rng(m * 7 + n)
    a = r.integers(-127, 128, size=(m, k)).astype(np.int8)
    b = r.integers(-127, 128, size=(n, k)).astype(np.int8)
    show("int8 acc", m, n, k)
    out = q.int8_gemm(to_dev_i8(a), to_dev_i8(b), None, None, out_dtype=torch.int32)
    assert np.array_equal(out.cpu().numpy().astype(np.int64), R.int8_accumulate(a, b))


def test_int32_accumulators_extreme_values(q):
    k = 133144 // 8 * 8
    a = np.full((3, k), -127, np.int8)
    b = np.full((5, k), 127, np.int8)
    b[1] = -127
    show("int8 acc extreme")
    out = q.int8_gemm(to_dev_i8(a), to_dev_i8(b), None, None, out_dtype=torch.int32)
    assert np.array_equal(out.cpu().numpy().astype(np.int64), R.int8_accumulate(a, b))


@pytest.mark.parametrize("n", [3072, 12288])
def test_w8a8_workload(q, n):
    c = synth.config5_case(n)
    qx, sx = R.int8_quantize_act(c.x)
    show("w8a8 workload", c.name)
    a_d, sa_d = q.int8_quantize_act(to_dev_bf16(c.x))
    b_d = to_dev_i8(c.b)
    sb_d = torch.from_numpy(c.b_scale).to(DEV)
    bias_d = to_dev_bf16(c.bias)
    out = q.int8_gemm(a_d, b_d, sa_d, sb_d, bias_d, out_dtype=torch.bfloat16)
    acc = q.int8_gemm(a_d, b_d, None, None, out_dtype=torch.int32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.random.default_rng(n).choice(c.x.shape[0], 256, replace=False),
                                     np.arange(c.x.shape[0] - 5, c.x.shape[0])]))
    want_acc = R.int8_accumulate(qx[rows], c.b)
    assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), want_acc)
    ref, tau = R.int8_epilogue(want_acc, sx[rows], c.b_scale, c.bias)
    res = C.check_bf16(bf16_bits(out)[rows], ref, tau)
    assert res and res.n_clause2 <= C.clause2_budget(ref), res


def test_epilogue_bf16_at_tile_edges(q):
    """bf16 epilogue at M = 4000, N = 3000: full 256 x 256 tiles leave through
    the LDS slab, edge tiles element by element."""
    r = np.random.default_rng(63)
    m, n, k = 4000, 3000, 512
    a = r.integers(-127, 128, size=(m, k)).astype(np.int8)
    b = r.integers(-127, 128, size=(n, k)).astype(np.int8)
    sa = (r.random(m).astype(np.float32) * 0.01).astype(np.float32)
    sb = (r.random(n).astype(np.float32) * 0.01).astype(np.float32)
    bias = synth.bf16_activation((64,), 1, n)[0]
    show("int8 epilogue bf16 edges")
    out = q.int8_gemm(to_dev_i8(a), to_dev_i8(b), torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV),
                      to_dev_bf16(bias), out_dtype=torch.bfloat16)
    ref, tau = R.int8_epilogue(R.int8_accumulate(a, b), sa, sb, bias)
    res = C.check_bf16(bf16_bits(out), ref, tau)
    assert res and res.n_clause2 <= C.clause2_budget(ref), res


def test_epilogue_without_bias_and_f32(q):
    r = np.random.default_rng(62)
    m, n, k = 200, 300, 512
    a = r.integers(-127, 128, size=(m, k)).astype(np.int8)
    b = r.integers(-127, 128, size=(n, k)).astype(np.int8)
    sa = (r.random(m).astype(np.float32) * 0.01).astype(np.float32)
    sb = (r.random(n).astype(np.float32) * 0.01).astype(np.float32)
    show("int8 epilogue f32")
    out = q.int8_gemm(to_dev_i8(a), to_dev_i8(b), torch.from_numpy(sa).to(DEV), torch.from_numpy(sb).to(DEV),
                      None, out_dtype=torch.float32)
    ref, tau = R.int8_epilogue(R.int8_accumulate(a, b), sa, sb)
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= tau)


def test_int8_rejects_bad_arguments(q):
    a = torch.zeros((2, 16), dtype=torch.int8, device=DEV)
    assert q.lib.qlinear_int8_gemm(a.data_ptr(), a.data_ptr(), None, None, None, a.data_ptr(), 1, 2, 2, 16,
                                   None) == q.ERR_INVALID_ARG  # bf16 output needs the scales
    assert q.lib.qlinear_int8_gemm(a.data_ptr(), a.data_ptr(), None, None, None, a.data_ptr(), 2, 2, 2, 133145,
                                   None) == q.ERR_INVALID_ARG  # K past the int32 range
