"""Seeded random-shape sweeps through the automatic kernel choice of every
call, on exact (dyadic) inputs, so that each output must equal the CPU
oracle's bit for bit: whatever kernel the shape lands on (GEMV, skinny,
split-K, tiled, register-staged, element-wise), with ragged M / N / K,
K not a multiple of 16 or 64, and weight views off a 16-byte boundary.
Integer work (int8 accumulators) is compared raw."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import ref as R
from gpu_util import DEV, bf16_bits, show, to_dev_bf16, to_dev_i8, to_dev_u8

pytestmark = pytest.mark.gpu

SEED = 20261202


@pytest.fixture(scope="module")
def q():
    import weight_quantized_linear_amd as q
    return q


def _rng(*key):
    return np.random.default_rng([SEED, *key])


def _m(r):
    # the dispatch bands: GEMV (M <= 4), skinny (<= 16), tiled
    band = r.integers(0, 3)
    return int(r.integers(1, 5) if band == 0 else r.integers(5, 17) if band == 1 else r.integers(17, 300))


def _k(r, lo=1, hi=3000):
    kind = r.integers(0, 3)  # multiple of 64, of 16, anything
    k = int(r.integers(lo, hi))
    return max(64, k // 64 * 64) if kind == 0 else max(16, k // 16 * 16) if kind == 1 else k


def _check(out, ref, out_dtype):
    if out_dtype == torch.float32:
        assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))
    else:
        assert np.array_equal(bf16_bits(out), F.f64_to_bf16_bits(ref))


def _weight_view(codes, offset):
    """A device copy of the [N, K] byte matrix that starts `offset` bytes past
    a 16-byte boundary; the bytes around it are NaN codes."""
    n, k = codes.shape
    flat = np.full(n * k + 32, 0x7F, np.uint8)
    flat[offset:offset + n * k] = codes.reshape(-1)
    return to_dev_u8(flat)[offset:offset + n * k].view(n, k)


@pytest.mark.parametrize("case", range(60))
def test_fp8_gemm_random_shapes(q, case):
    r = _rng(1, case)
    m, n, k = _m(r), int(r.integers(1, 1500)), _k(r)
    offset = int(r.integers(1, 16)) if r.integers(0, 3) == 0 else 0
    out_dtype = torch.float32 if case % 2 else torch.bfloat16
    wc = synth.dyadic_fp8_weight((70, case), n, k)
    xc = synth.dyadic_activation((71, case), m, k)
    ref, _ = R.fp8_linear(wc, xc)
    show("sweep fp8", m, n, k, offset, out_dtype)
    out = q.fp8_gemm(_weight_view(wc, offset), to_dev_bf16(xc), out_dtype=out_dtype)
    _check(out, ref, out_dtype)


@pytest.mark.parametrize("case", range(24))
def test_fp8_gemm_random_long_k(q, case):
    """The split-K region of the automatic choice (a workspace is given):
    K >= 8192 made of 2048-value slices (the streaming kernel's split-K form)
    or any other multiple of 64 (the split-K skinny kernel), M = 2..16 and
    N from 16 to 12000 (ragged 16-row tiles)."""
    r = _rng(8, case)
    m, n = int(r.integers(2, 17)), int(r.integers(16, 12001))
    k = 2048 * int(r.integers(4, 9)) if case % 3 else 64 * int(r.integers(128, 257))
    out_dtype = torch.float32 if case % 2 else torch.bfloat16
    wc = synth.dyadic_fp8_weight((72, case), n, k)
    xc = synth.dyadic_activation((73, case), m, k)
    ref, _ = R.fp8_linear(wc, xc)
    show("sweep fp8 long K", m, n, k, out_dtype)
    out = q.fp8_gemm(to_dev_u8(wc), to_dev_bf16(xc), out_dtype=out_dtype)
    _check(out, ref, out_dtype)


@pytest.mark.parametrize("case", range(32))
def test_nvfp4_gemm_random_shapes(q, case):
    r = _rng(2, case)
    m, n, k = _m(r), int(r.integers(1, 1500)), 16 * int(r.integers(1, 190))
    out_dtype = torch.float32 if case % 2 else torch.bfloat16
    packed, scales = synth.dyadic_nvfp4_weight((72, case), n, k)
    xc = synth.dyadic_activation((73, case), m, k)
    ref, _ = R.nvfp4_linear(packed, scales, xc)
    show("sweep nvfp4", m, n, k, out_dtype)
    out = q.nvfp4_gemm(to_dev_u8(packed), to_dev_u8(scales), to_dev_bf16(xc), out_dtype=out_dtype)
    _check(out, ref, out_dtype)


@pytest.mark.parametrize("case", range(24))
def test_bf16_gemm_random_shapes(q, case):
    r = _rng(3, case)
    m, n, k = _m(r), int(r.integers(1, 1500)), _k(r)
    out_dtype = torch.float32 if case % 2 else torch.bfloat16
    wb = synth.dyadic_bf16_weight((74, case), n, k)
    xb = synth.dyadic_activation((75, case), m, k)
    ref, _ = R.bf16_linear(wb, xb)
    show("sweep bf16", m, n, k, out_dtype)
    out = q.bf16_gemm(to_dev_bf16(wb), to_dev_bf16(xb), out_dtype=out_dtype)
    _check(out, ref, out_dtype)


@pytest.mark.parametrize("case", range(24))
def test_int8_accumulators_random_shapes(q, case):
    r = _rng(4, case)
    m, n, k = int(r.integers(1, 600)), int(r.integers(1, 1500)), _k(r)
    a = r.integers(-127, 128, size=(m, k)).astype(np.int8)
    b = r.integers(-127, 128, size=(n, k)).astype(np.int8)
    show("sweep int8", m, n, k)
    out = q.int8_gemm(to_dev_i8(a), to_dev_i8(b), None, None, out_dtype=torch.int32)
    assert np.array_equal(out.cpu().numpy().astype(np.int64), R.int8_accumulate(a, b))


@pytest.mark.parametrize("case", range(24))
def test_fp8_w8a8_random_shapes(q, case):
    r = _rng(5, case)
    m, n, k = int(r.integers(1, 600)), int(r.integers(1, 1500)), _k(r)
    out_dtype = torch.float32 if case % 2 else torch.bfloat16
    xq = synth.dyadic_e4m3_activation((76, case), m, k)
    w = synth.dyadic_fp8_weight((77, case), n, k)
    ref, _ = R.fp8_w8a8_linear(xq, w, 0.25)
    show("sweep w8a8", m, n, k, out_dtype)
    out = q.fp8_w8a8_gemm(to_dev_u8(xq), to_dev_u8(w), out_dtype=out_dtype, alpha=0.25)
    _check(out, ref, out_dtype)


def _groups(r, t, e):
    """Non-decreasing offsets inside [0, t] (rows before the first and after
    the last group uncovered), empty groups, ids with -1."""
    g = int(r.integers(1, 10))
    cuts = np.sort(r.integers(0, t + 1, size=g + 1))
    ids = r.integers(-1, e, size=g).astype(np.int32)
    return cuts.astype(np.int64), ids


@pytest.mark.parametrize("case", range(16))
def test_grouped_random_shapes(q, case):
    r = _rng(6, case)
    e, n, t = int(r.integers(1, 7)), int(r.integers(1, 600)), int(r.integers(1, 500))
    k = _k(r, 16, 2500)
    offs, ids = _groups(r, t, e)
    # W8A16 experts
    w = synth.dyadic_fp8_weight((78, case), e * n, k).reshape(e, n, k)
    x = synth.dyadic_activation((79, case), t, k)
    ref, _, written = R.fp8_grouped(w, x, offs, ids)
    show("sweep grouped fp8", e, n, t, k, offs.tolist(), ids.tolist())
    out = torch.full((t, n), float("nan"), dtype=torch.float32, device=DEV)
    q.fp8_grouped_gemm(to_dev_u8(w), to_dev_bf16(x), torch.from_numpy(offs.astype(np.int32)).to(DEV),
                       torch.from_numpy(ids).to(DEV), out=out, out_dtype=torch.float32)
    got = out.cpu().numpy()
    assert np.array_equal(got[written], ref[written].astype(np.float32))
    assert np.all(np.isnan(got[~written]))
    # int8 experts, raw accumulators
    a = r.integers(-127, 128, size=(t, k)).astype(np.int8)
    b = r.integers(-127, 128, size=(e, n, k)).astype(np.int8)
    acc, _, written = R.int8_grouped(a, b, None, None, None, offs, ids, raw=True)
    show("sweep grouped int8", e, n, t, k)
    raw = torch.full((t, n), -7, dtype=torch.int32, device=DEV)
    q.int8_grouped_gemm(to_dev_i8(a), to_dev_i8(b), None, None, torch.from_numpy(offs.astype(np.int32)).to(DEV),
                        torch.from_numpy(ids).to(DEV), out=raw, out_dtype=torch.int32)
    g = raw.cpu().numpy()
    assert np.array_equal(g[written], acc[written].astype(np.int32))
    assert np.all(g[~written] == -7)
    # NVFP4 experts (K a multiple of 16)
    k4 = max(16, k // 16 * 16)
    p, s = synth.dyadic_nvfp4_weight((80, case), e * n, k4)
    p, s = p.reshape(e, n, k4 // 2), s.reshape(e, n, k4 // 16)
    x4 = synth.dyadic_activation((81, case), t, k4)
    ref4, _, written = R.nvfp4_grouped(p, s, x4, offs, ids)
    show("sweep grouped nvfp4", e, n, t, k4)
    out4 = torch.full((t, n), float("nan"), dtype=torch.float32, device=DEV)
    q.nvfp4_grouped_gemm(to_dev_u8(p), to_dev_u8(s), to_dev_bf16(x4), torch.from_numpy(offs.astype(np.int32)).to(DEV),
                         torch.from_numpy(ids).to(DEV), out=out4, out_dtype=torch.float32)
    g4 = out4.cpu().numpy()
    assert np.array_equal(g4[written], ref4[written].astype(np.float32))
    assert np.all(np.isnan(g4[~written]))


@pytest.mark.parametrize("g", [65, 129, 200])
def test_grouped_many_groups(q, g):
    """More groups than one wave's 64 lanes: the kernels' prefix sum of the
    groups' row tiles carries across several passes (exact inputs, every
    family bit for bit; empty, inactive and uncovered rows included)."""
    r = _rng(7, g)
    e, n, k, t = 8, 136, 256, 900
    cuts = np.sort(r.integers(0, t + 1, size=g + 1)).astype(np.int64)
    ids = r.integers(-1, e, size=g).astype(np.int32)
    offs_dev = torch.from_numpy(cuts.astype(np.int32)).to(DEV)
    ids_dev = torch.from_numpy(ids).to(DEV)
    w = synth.dyadic_fp8_weight((82, g), e * n, k).reshape(e, n, k)
    x = synth.dyadic_activation((83, g), t, k)
    ref, _, written = R.fp8_grouped(w, x, cuts, ids)
    show("many groups fp8", g, e, n, t, k)
    out = torch.full((t, n), float("nan"), dtype=torch.float32, device=DEV)
    q.fp8_grouped_gemm(to_dev_u8(w), to_dev_bf16(x), offs_dev, ids_dev, out=out, out_dtype=torch.float32)
    got = out.cpu().numpy()
    assert np.array_equal(got[written], ref[written].astype(np.float32))
    assert np.all(np.isnan(got[~written]))
    a = r.integers(-127, 128, size=(t, k)).astype(np.int8)
    b = r.integers(-127, 128, size=(e, n, k)).astype(np.int8)
    acc, _, written = R.int8_grouped(a, b, None, None, None, cuts, ids, raw=True)
    show("many groups int8", g)
    raw = torch.full((t, n), -7, dtype=torch.int32, device=DEV)
    q.int8_grouped_gemm(to_dev_i8(a), to_dev_i8(b), None, None, offs_dev, ids_dev, out=raw, out_dtype=torch.int32)
    gi = raw.cpu().numpy()
    assert np.array_equal(gi[written], acc[written].astype(np.int32))
    assert np.all(gi[~written] == -7)
    p, s = synth.dyadic_nvfp4_weight((84, g), e * n, k)
    p, s = p.reshape(e, n, k // 2), s.reshape(e, n, k // 16)
    ref4, _, written = R.nvfp4_grouped(p, s, x, cuts, ids)
    show("many groups nvfp4", g)
    out4 = torch.full((t, n), float("nan"), dtype=torch.float32, device=DEV)
    q.nvfp4_grouped_gemm(to_dev_u8(p), to_dev_u8(s), to_dev_bf16(x), offs_dev, ids_dev, out=out4,
                         out_dtype=torch.float32)
    g4 = out4.cpu().numpy()
    assert np.array_equal(g4[written], ref4[written].astype(np.float32))
    assert np.all(np.isnan(g4[~written]))
