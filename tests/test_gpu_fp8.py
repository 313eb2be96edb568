"""GPU parity of the W8A16 calls (GEMV, skinny, materialize) against the
CPU oracle, through the C ABI."""

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


def _no_nan_codes(r, shape):
    w = r.integers(0, 256, size=shape, dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38
    return w


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("n,k", [(2, 128), (1, 255), (3, 1)])
def test_materialize_every_code_bit_exact(q, n, k):
    codes = (np.arange(n * k) % 256).astype(np.uint8).reshape(n, k)
    want = F.e4m3_to_f64(codes)
    nan = np.isnan(want)
    w = to_dev_u8(codes)
    show("materialize f32", n, k)
    got = q.fp8_materialize(w, torch.float32).cpu().numpy()
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].astype(np.float32).view(np.uint32))
    show("materialize bf16", n, k)
    gb = bf16_bits(q.fp8_materialize(w, torch.bfloat16))
    assert np.array_equal((gb & 0x7FFF) > 0x7F80, nan)
    assert np.array_equal(gb[~nan], F.f64_to_bf16_bits(want[~nan]))


def test_gemv_one_hot_returns_decoded_column(q):
    r = np.random.default_rng(1)
    codes = _no_nan_codes(r, (300, 4096))
    w = to_dev_u8(codes)
    dec = F.e4m3_to_f64(codes)
    for k in (0, 17, 2049, 4095):
        x = np.zeros((1, 4096), np.uint16)
        x[0, k] = 0x3F80
        show("gemv one-hot", k)
        got = q.fp8_gemv(w, to_dev_bf16(x[0]), out_dtype=torch.float32).cpu().numpy()
        assert np.array_equal(got.astype(np.float64), dec[:, k])


# ------------------------------------------------------------------ exact (dyadic) inputs

DYADIC = [
    ("gemv", 1, 1, 16), ("gemv", 1, 7, 4096), ("gemv", 1, 515, 2050), ("gemv", 1, 33, 3),
    ("gemv", 1, 260, 14336), ("gemv", 1, 129, 1000), ("gemv", 2, 129, 2064), ("gemv", 3, 5, 48),
    ("gemv", 4, 1031, 4096), ("gemv", 4, 70, 2050),
    ("skinny", 1, 17, 16), ("skinny", 2, 300, 64), ("skinny", 4, 1000, 4096), ("skinny", 5, 33, 4112),
    ("skinny", 16, 1000, 1040), ("skinny", 16, 4111, 4096), ("skinny", 11, 2000, 14336),
    ("auto", 16, 4096, 4096),
    # wide-N skinny kernels (4x4x4 matrix-core path for M <= 4, LDS-staged path for M > 4)
    ("skinny", 4, 65600, 64), ("auto", 3, 70000, 256), ("skinny", 16, 65601, 528), ("auto", 7, 66000, 1024),
    # activation-in-LDS skinny kernel (K % 256 == 0): ragged N, every m-group size, partial last
    # stage of 16 chunks, the largest K each m-group accepts, and small N on few blocks
    ("skinny", 1, 4097, 4352), ("skinny", 8, 1001, 512), ("skinny", 9, 333, 5120),
    ("skinny", 2, 150, 10240), ("skinny", 13, 70001, 256), ("skinny", 4, 7, 19712),
    ("skinny", 12, 66003, 4096), ("skinny", 5, 1, 256),
    # 16x16x32 activation-in-LDS kernel (5 <= M <= 16, K % 64 == 0): the largest K, uneven K split
    ("skinny", 16, 300, 4864), ("skinny", 6, 2050, 4800),
    # split-K skinny kernel: K slices of 64-value chunks with a ragged last slice, fewer columns than
    # one block, every M, and the automatic choice at M = 12, K = 8192
    ("splitk", 16, 4096, 14336), ("splitk", 3, 1000, 4096), ("splitk", 9, 300, 2112), ("splitk", 16, 70, 1024),
    ("splitk", 1, 129, 512), ("auto", 12, 2000, 8192),
    # its streaming form where K is made of 2048-value slices (two to eight slices): the smallest N,
    # a ragged last 16-row tile, several tiles per block
    ("splitk", 1, 16, 4096), ("splitk", 16, 4111, 6144), ("splitk", 5, 20000, 16384), ("splitk", 4, 4096, 14336),
    # the automatic choice takes it from M = 3, and at M = 2 from 8192 output features
    ("auto", 2, 8192, 8192), ("auto", 3, 4096, 14336), ("auto", 2, 4096, 14336),
    # streaming skinny kernel (K in {1024, 2048, 3072, 4096}; N >= 6144 for 5 <= M <= 16, 8192 <= N <
    # 65536 for M = 3, and for M = 4 also 4096 <= N < 8192 at K = 4096): every ring depth, a ragged
    # last 16-row tile, every M class, the smallest N it takes (fewer tiles than blocks on some CUs,
    # one stage on a block), M = 3, 4 below the 4x4x4 kernel's range
    ("skinny", 16, 65553, 2048), ("skinny", 5, 65536, 3072), ("auto", 9, 65537, 1024),
    ("skinny", 16, 131087, 4096), ("auto", 6, 100003, 4096),
    ("auto", 16, 14336, 4096), ("auto", 3, 8192, 1024), ("auto", 4, 14343, 2048), ("skinny", 5, 8197, 3072),
    ("auto", 4, 4096, 4096), ("auto", 4, 4111, 4096), ("auto", 16, 6144, 4096), ("auto", 8, 6150, 1024),
    ("skinny", 5, 6144, 2048),
]


@pytest.mark.parametrize("path,m,n,k", DYADIC)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dyadic_inputs_are_bit_exact(q, path, m, n, k, out_dtype):
    wc = synth.dyadic_fp8_weight((10, m, n, k), n, k)
    xc = synth.dyadic_activation((11, m, n, k), m, k)
    ref, _ = R.fp8_linear(wc, xc)
    show("dyadic", path, m, n, k, out_dtype)
    out = q.fp8_gemm(to_dev_u8(wc), to_dev_bf16(xc), out_dtype=out_dtype, path=path)
    if out_dtype == torch.float32:
        assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))
    else:
        assert np.array_equal(bf16_bits(out), F.f64_to_bf16_bits(ref))


# GEMV weight rows at any byte offset (K % 16 != 0, or a weight view that
# starts off a 16-byte boundary): 16-byte loads shifted into place.  One and
# two rows per wave, one and several passes over K, K below one chunk.  The
# bytes around the view are NaN codes, so a byte read past a row's end and not
# cleared shows up as NaN.
@pytest.mark.parametrize("m,n,k", [(1, 515, 2050), (1, 4100, 2050), (1, 70, 4100), (2, 300, 1000),
                                   (3, 70, 24), (1, 64, 7), (4, 4097, 4096)])
@pytest.mark.parametrize("offset", [0, 1, 6, 15])
def test_gemv_weight_rows_at_any_offset(q, m, n, k, offset):
    wc = synth.dyadic_fp8_weight((14, m, n, k), n, k)
    xc = synth.dyadic_activation((15, m, n, k), m, k)
    ref, _ = R.fp8_linear(wc, xc)
    flat = np.full(n * k + 32, 0x7F, np.uint8)
    flat[offset:offset + n * k] = wc.reshape(-1)
    w = to_dev_u8(flat)[offset:offset + n * k].view(n, k)
    show("gemv weight offset", m, n, k, offset)
    out = q.fp8_gemm(w, to_dev_bf16(xc), out_dtype=torch.float32, path="gemv")
    assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))


# An activation that starts off a 16-byte boundary takes the byte-load kernel.
@pytest.mark.parametrize("m,k", [(1, 2050), (2, 4096)])
def test_gemv_unaligned_activation(q, m, k):
    n = 300
    wc = synth.dyadic_fp8_weight((16, m, k), n, k)
    xc = synth.dyadic_activation((17, m, k), m, k)
    ref, _ = R.fp8_linear(wc, xc)
    xbuf = to_dev_bf16(np.concatenate([np.zeros(1, xc.dtype), xc.reshape(-1)]))
    x = xbuf[1:].view(m, k)
    assert x.data_ptr() % 16 != 0
    show("gemv unaligned x", m, k)
    out = q.fp8_gemm(to_dev_u8(wc), x, out_dtype=torch.float32, path="gemv")
    assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_gemv_and_skinny_agree_on_exact_inputs(q, m):
    wc = synth.dyadic_fp8_weight((12, m), 777, 4096)
    xc = synth.dyadic_activation((13, m), m, 4096)
    w, x = to_dev_u8(wc), to_dev_bf16(xc)
    show("cross-path", m)
    a = q.fp8_gemm(w, x, out_dtype=torch.float32, path="gemv")
    b = q.fp8_gemm(w, x, out_dtype=torch.float32, path="skinny")
    assert torch.equal(a, b)


# ------------------------------------------------------------------ the GEMV workload (M = 1, N = 2048)

@pytest.mark.parametrize("case", [0, 1])
def test_gemv_n2048_raw_and_scale_fold(q, case):
    c = synth.config1_case(case)
    ref, bound = R.fp8_linear(c.w, c.x)
    w, x = to_dev_u8(c.w), to_dev_bf16(c.x[0])
    show("gemv n2048", c.name)
    raw = q.fp8_gemv(w, x, out_dtype=torch.float32).cpu().numpy()
    res = C.check_f32(raw[None, :], ref, bound)
    assert res, res
    assert res.max_rel < 1e-5, res  # ~sqrt(K) * 2^-24 expected
    # fold: alpha applied in float32 to the same accumulation
    scaled = q.fp8_gemv(w, x, out_dtype=torch.float32, alpha=c.alpha).cpu().numpy()
    assert np.array_equal(scaled, (raw * np.float32(c.alpha)).astype(np.float32))
    ref_a, bound_a = R.fp8_linear(c.w, c.x, c.alpha)
    assert C.check_f32(scaled[None, :], ref_a, bound_a)


# ------------------------------------------------------------------ decode GEMV / skinny workload

@pytest.fixture(scope="module")
def config2_weights():
    cache = {}

    def get(idx):
        if idx not in cache:
            n, k = synth.CONFIG2_SHAPES[idx]
            codes, s = synth.fp8_weight((2, idx, 0), n, k)
            cache[idx] = (codes, s, to_dev_u8(codes))
        return cache[idx]
    return get


@pytest.mark.parametrize("shape_idx", [0, 1, 2, 3])
@pytest.mark.parametrize("m", synth.CONFIG2_M)
def test_decode_workload_bf16(q, config2_weights, shape_idx, m):
    codes, s, w = config2_weights(shape_idx)
    c = synth.config2_case(shape_idx, m, weight=(codes, s))
    n, k = codes.shape
    show("decode workload", c.name)
    out = q.fp8_gemm(w, to_dev_bf16(c.x), out_dtype=torch.bfloat16, alpha=c.alpha)
    torch.cuda.synchronize()
    got = bf16_bits(out)
    if n > 20000:  # sample rows the oracle computes one by one, plus the ragged end
        rows = np.unique(np.concatenate([np.random.default_rng(shape_idx).choice(n, 3000, replace=False),
                                         np.arange(n - 70, n), np.arange(0, 64)]))
    else:
        rows = np.arange(n)
    ref, bound = R.fp8_linear(codes[rows], c.x, c.alpha)
    res = C.check_bf16(got[:, rows], ref, C.fp_tolerance(bound))
    assert res, res
    assert res.n_clause2 <= C.clause2_budget(ref), res


# ------------------------------------------------------------------ hygiene

@pytest.mark.parametrize("path,m", [("gemv", 1), ("gemv", 3), ("skinny", 7)])
def test_writes_stay_inside_out(q, path, m):
    n, k = 333, 1024
    r = np.random.default_rng(5)
    wc = _no_nan_codes(r, (n, k))
    xc = synth.bf16_activation((9, m), m, k)
    buf = torch.full((m * n + 4096,), float("nan"), dtype=torch.float32, device="cuda:0")
    show("stray", path, m)
    q.fp8_gemm(to_dev_u8(wc), to_dev_bf16(xc), out=buf[: m * n].view(m, n), out_dtype=torch.float32, path=path)
    tail = buf[m * n:].cpu().numpy()
    assert np.all(np.isnan(tail))
    assert not np.any(np.isnan(buf[: m * n].cpu().numpy()))


@pytest.mark.parametrize("m", [1, 4, 16])
def test_repeat_runs_are_bitwise_identical(q, m):
    codes, _ = synth.fp8_weight((20, m), 5000, 4096)
    xc = synth.bf16_activation((21, m), m, 4096)
    w, x = to_dev_u8(codes), to_dev_bf16(xc)
    show("determinism", m)
    a = q.fp8_gemm(w, x, out_dtype=torch.float32)
    b = q.fp8_gemm(w, x, out_dtype=torch.float32)
    assert torch.equal(a, b)


def test_gemm_rejects_mismatched_shapes(q):
    w = torch.zeros((8, 16), dtype=torch.uint8, device="cuda:0")
    x = torch.zeros((2, 32), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ValueError):
        q.fp8_gemm(w, x)


def test_splitk_reports_unsuitable_shapes(q):
    """A K too short for two slices gives QLINEAR_ERR_UNSUPPORTED and launches
    nothing; the automatic choice takes the skinny kernel instead."""
    wc = synth.dyadic_fp8_weight((14,), 70000, 256)
    xc = synth.dyadic_activation((15,), 12, 256)
    w, x = to_dev_u8(wc), to_dev_bf16(xc)
    out = torch.full((12, 70000), 7.0, dtype=torch.float32, device="cuda:0")
    show("splitk unsuitable")
    with pytest.raises(q.QLinearError) as e:
        q.fp8_gemm(w, x, out=out, out_dtype=torch.float32, path="splitk")
    assert e.value.status == q.ERR_UNSUPPORTED
    assert torch.all(out == 7.0)
    w2 = to_dev_u8(synth.dyadic_fp8_weight((16,), 100, 208))  # K % 64 != 0
    x2 = to_dev_bf16(synth.dyadic_activation((17,), 12, 208))
    with pytest.raises(q.QLinearError) as e:
        q.fp8_gemm(w2, x2, out_dtype=torch.float32, path="splitk")
    assert e.value.status == q.ERR_INVALID_ARG
