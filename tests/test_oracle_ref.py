"""Pins of the oracle's reference results (oracle.ref): hand-worked examples
(tests/golden), exact rational brute force on tiny inputs, exact integer
brute force, the scale-fold invariant and special cases with known answers."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import formats as F
from oracle import ref as R
import synth


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _hex_array(rows, dtype):
    return np.array([[int(v, 16) for v in r] for r in rows], dtype=dtype)


# ------------------------------------------------------------------ W8A16

def test_fp8_linear_golden():
    g = _load("fp8_linear_example.json")
    w = _hex_array(g["w_codes"], np.uint8)
    x = _hex_array(g["x_bits"], np.uint16)
    assert np.array_equal(F.e4m3_to_f64(w), np.array(g["w_values"], float))
    assert np.array_equal(F.bf16_bits_to_f64(x), np.array(g["x_values"], float))
    raw, bound = R.fp8_linear(w, x)
    assert np.array_equal(raw, np.array(g["raw"], float))
    assert np.array_equal(bound, np.array(g["bound"], float))
    scaled, _ = R.fp8_linear(w, x, float(g["alpha"]))
    assert np.array_equal(scaled, np.array(g["scaled"], float))
    assert np.array_equal(F.f64_to_bf16_bits(raw), _hex_array(g["raw_bf16_bits"], np.uint16))


def _fraction_linear(wvals, xvals):
    m, k = xvals.shape
    n = wvals.shape[0]
    out = [[sum((Fraction(float(xvals[i, t])) * Fraction(float(wvals[j, t])) for t in range(k)), Fraction(0))
            for j in range(n)] for i in range(m)]
    return out


@pytest.mark.parametrize("m,n,k", [(1, 3, 5), (2, 5, 7), (3, 4, 33), (5, 2, 1)])
def test_fp8_linear_fraction_brute_force(m, n, k):
    r = np.random.default_rng(m * 100 + n * 10 + k)
    w = r.integers(0, 256, size=(n, k), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38                    # no NaN codes
    x = synth.bf16_bits_from_f32(r.standard_normal((m, k)).astype(np.float32))
    got, bound = R.fp8_linear(w, x)
    exact = _fraction_linear(F.e4m3_to_f64(w), F.bf16_bits_to_f64(x))
    for i in range(m):
        for j in range(n):
            e = exact[i][j]
            assert abs(Fraction(float(got[i, j])) - e) <= Fraction(2.0 ** -40) * Fraction(float(bound[i, j])) + Fraction(2.0 ** -1000)
    assert got.shape == (m, n)


def test_fp8_linear_one_hot_activation_returns_decoded_column():
    """x = e_k selects column k of dec(W): out[n] = dec(W[n, k]) exactly (a
    NaN code anywhere in row n makes out[n] NaN, since NaN * 0 is NaN)."""
    w = np.arange(256, dtype=np.uint8).reshape(16, 16)
    w[:, 15] = 0x38                                 # keep NaN codes out of the other columns' rows
    w[7, 3], w[15, 3] = 0x7F, 0xFF
    for k in (0, 3, 5, 14):
        x = np.zeros((1, 16), np.uint16)
        x[0, k] = 0x3F80                           # bf16 1.0
        out, _ = R.fp8_linear(w, x)
        col = F.e4m3_to_f64(w[:, k])
        nan = np.isnan(F.e4m3_to_f64(w)).any(axis=1)
        assert np.array_equal(np.isnan(out[0]), nan)
        assert np.array_equal(out[0][~nan], col[~nan])


def test_fp8_scale_fold_invariant():
    """fp8_gemv page, 'Scale contract': a scalar weight_scale factors out of the
    sum.  ref(alpha) == alpha * ref(1), bit-equal for powers of two and
    within float64 rounding otherwise."""
    c = synth.config1_case(0)
    w, x = c.w[:64], c.x
    raw, b1 = R.fp8_linear(w, x)
    for a in (0.5, 2.0 ** -12, 8.0):
        got, b = R.fp8_linear(w, x, a)
        assert np.array_equal(got, a * raw) and np.array_equal(b, a * b1)
    got, _ = R.fp8_linear(w, x, c.alpha)
    assert np.allclose(got, c.alpha * raw, rtol=1e-15, atol=0)


def test_fp8_linear_chunking_is_transparent(monkeypatch):
    r = np.random.default_rng(3)
    w = r.integers(0, 0x7E, size=(50, 40), dtype=np.uint8)
    x = synth.bf16_bits_from_f32(r.standard_normal((3, 40)).astype(np.float32))
    full, bf = R.fp8_linear(w, x)
    monkeypatch.setattr(R, "_ROW_CHUNK", 7)
    chunked, bc = R.fp8_linear(w, x)
    assert np.array_equal(full, chunked) and np.array_equal(bf, bc)


# ------------------------------------------------------------------ grouped

def _tiny_grouped(seed=11, e=4, n=6, k=9, t=13):
    r = np.random.default_rng(seed)
    w = r.integers(0, 0x7E, size=(e, n, k), dtype=np.uint8)
    x = synth.bf16_bits_from_f32(r.standard_normal((t, k)).astype(np.float32))
    return w, x


def test_grouped_brute_force_and_semantics():
    w, x = _tiny_grouped()
    offs = np.array([0, 3, 3, 7, 9, 12], np.uint32)   # group 1 empty, row 12 uncovered
    ids = np.array([2, 0, -1, 1, 3], np.int32)
    ref, bound, written = R.fp8_grouped(w, x, offs, ids)
    assert written.tolist() == [True] * 12 + [False]
    assert np.all(np.isnan(ref[12]))
    assert np.array_equal(ref[3:7], np.zeros((4, 6)))            # id -1 -> zeros
    wd = F.e4m3_to_f64(w)
    xd = F.bf16_bits_to_f64(x)
    for rows, ex in (((0, 3), 2), ((7, 9), 1), ((9, 12), 3)):
        exact = _fraction_linear(wd[ex], xd[rows[0]:rows[1]])
        for i in range(rows[1] - rows[0]):
            for j in range(6):
                assert abs(Fraction(float(ref[rows[0] + i, j])) - exact[i][j]) <= Fraction(2.0 ** -40) * Fraction(float(bound[rows[0] + i, j]) + 1)


def test_grouped_single_group_equals_dense():
    w, x = _tiny_grouped(seed=5)
    ref, _, written = R.fp8_grouped(w, x, np.array([0, 13], np.uint32), np.array([1], np.int32))
    dense, _ = R.fp8_linear(w[1], x)
    assert written.all() and np.array_equal(ref, dense)


def test_grouped_guard_readings():
    """Out-of-range ids behave as -1; a decreasing offset pair is empty; rows
    past T are clipped."""
    w, x = _tiny_grouped(seed=6)
    offs = np.array([0, 2, 1, 5, 40], np.uint32)
    ids = np.array([7, 0, -5, 1], np.int32)
    ref, _, written = R.fp8_grouped(w, x, offs, ids)
    assert np.array_equal(ref[0:2], np.zeros((2, 6)))           # id 7 >= E -> zeros
    assert np.array_equal(ref[1:5], np.zeros((4, 6)))           # id -5 -> zeros; [2,1) empty
    dense, _ = R.fp8_linear(w[1], x[5:13])
    assert np.array_equal(ref[5:13], dense) and written.all()


# ------------------------------------------------------------------ NVFP4

def test_nvfp4_dequant_golden():
    g = _load("nvfp4_dequant_example.json")
    p = _hex_array(g["packed"], np.uint8)
    s = _hex_array(g["scales"], np.uint8)
    d = R.nvfp4_dequant(p, s)
    want = np.array(g["expected"], float)
    assert np.array_equal(d, want) and np.array_equal(np.signbit(d), np.signbit(want))


def test_nvfp4_identity_activation_gives_transposed_dequant():
    """X = I_K: out = D^T (each output is one exact product)."""
    p, s, _ = synth.nvfp4_weight((99, 1), 5, 32)
    eye = synth.bf16_bits_from_f32(np.eye(32, dtype=np.float32))
    out, _ = R.nvfp4_linear(p, s, eye)
    assert np.array_equal(out, R.nvfp4_dequant(p, s).T)


@pytest.mark.parametrize("m,n,k", [(1, 2, 16), (3, 4, 48)])
def test_nvfp4_linear_fraction_brute_force(m, n, k):
    r = np.random.default_rng(k)
    codes = r.integers(0, 16, size=(n, k)).astype(np.uint8)
    p = synth.pack_nibbles(codes)
    s = r.integers(0, 0x7E, size=(n, k // 16), dtype=np.uint8)
    x = synth.bf16_bits_from_f32(r.standard_normal((m, k)).astype(np.float32))
    got, bound = R.nvfp4_linear(p, s, x, 0.75)
    # first principles: value(code) * value(scale), no shared helper beyond the pinned decoders
    e2 = F.e2m1_to_f64(np.arange(16))
    e4 = F.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    xd = F.bf16_bits_to_f64(x)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for t in range(k):
                byte = int(p[j, t // 2])
                nib = byte & 0xF if t % 2 == 0 else byte >> 4
                acc += Fraction(float(xd[i, t])) * Fraction(float(e2[nib])) * Fraction(float(e4[s[j, t // 16]]))
            assert abs(Fraction(float(got[i, j])) - Fraction(3, 4) * acc) <= Fraction(2.0 ** -40) * Fraction(float(bound[i, j]) + 1)


def test_nvfp4_grouped_brute_force_and_semantics():
    """Grouped NVFP4: each active group equals exact rational sums of
    x * e2m1(code) * e4m3(block scale) with its expert's weight; -1 groups are
    zeros, empty groups and uncovered rows are untouched."""
    r = np.random.default_rng(21)
    e_count, n, k, t = 3, 4, 32, 11
    codes = r.integers(0, 16, size=(e_count, n, k)).astype(np.uint8)
    packed = np.stack([synth.pack_nibbles(codes[e]) for e in range(e_count)])
    scales = r.integers(0, 0x7E, size=(e_count, n, k // 16), dtype=np.uint8)
    x = synth.bf16_bits_from_f32(r.standard_normal((t, k)).astype(np.float32))
    offs = np.array([0, 2, 2, 5, 7, 10], np.uint32)   # group 1 empty, row 10 uncovered
    ids = np.array([1, 0, -1, 2, 0], np.int32)
    ref, bound, written = R.nvfp4_grouped(packed, scales, x, offs, ids)
    assert written.tolist() == [True] * 10 + [False]
    assert np.all(np.isnan(ref[10]))
    assert np.array_equal(ref[2:5], np.zeros((3, n)))
    e2 = F.e2m1_to_f64(np.arange(16))
    e4 = F.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    xd = F.bf16_bits_to_f64(x)
    for (lo, hi), ex in (((0, 2), 1), ((5, 7), 2), ((7, 10), 0)):
        for i in range(lo, hi):
            for j in range(n):
                acc = Fraction(0)
                for kk in range(k):
                    acc += (Fraction(float(xd[i, kk])) * Fraction(float(e2[codes[ex, j, kk]]))
                            * Fraction(float(e4[scales[ex, j, kk // 16]])))
                assert abs(Fraction(float(ref[i, j])) - acc) <= Fraction(2.0 ** -40) * Fraction(float(bound[i, j]) + 1)


def test_nvfp4_rejects_bad_block_layout():
    with pytest.raises(ValueError):
        R.nvfp4_dequant(np.zeros((2, 8), np.uint8), np.zeros((2, 2), np.uint8))


# ------------------------------------------------------------------ int8

def test_int8_quantize_golden():
    g = _load("int8_example.json")["quantize"]
    xv = np.array(g["x_values"], dtype=np.float64)
    bits = F.f64_to_bf16_bits(xv)
    assert np.array_equal(F.bf16_bits_to_f64(bits), xv)       # values are bf16-exact
    q, s = R.int8_quantize_act(bits)
    assert np.array_equal(q, np.array(g["q"], np.int8))
    assert s.view(np.uint32).tolist() == [int(h, 16) for h in g["a_scale_bits"]]


def test_int8_quantize_properties():
    c = synth.config5_case(3072, m=64)
    q, s = R.int8_quantize_act(c.x)
    x = F.bf16_bits_to_f64(c.x)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127)
    am = np.abs(x).max(axis=1)
    assert np.array_equal(s, (am.astype(np.float32) / np.float32(127)).astype(np.float32))
    # the row absmax maps to +-127
    idx = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(q[np.arange(64), idx].astype(int)) == 127)
    # reconstruction error within half a step (plus float32 slack)
    err = np.abs(x - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 2.0 ** -17))


def test_int8_quantize_zero_and_ties():
    bits = F.f64_to_bf16_bits(np.array([[0.0, -0.0, 0.0], [127.0, 0.5, -1.5]]))
    q, s = R.int8_quantize_act(bits)
    assert s[0] == 0 and np.all(q[0] == 0)
    assert s[1] == 1.0 and q[1].tolist() == [127, 0, -2]


def test_int8_quantize_non_finite_rows():
    """Reading for inputs outside the workloads: the row formulas applied as
    written -- a NaN makes absmax and a_scale NaN, an infinity makes them
    +inf -- and such a row's codes are all zero, so the dequantised output
    of the row is NaN in every column."""
    nan, inf = float("nan"), float("inf")
    rows = np.array([[1.0, nan, -3.0, 2.0], [1.0, inf, -3.0, 2.0], [-inf, 0.5, 4.0, 0.0],
                     [inf, nan, 1.0, 1.0], [127.0, 1.0, -2.5, 0.0]])
    q, s = R.int8_quantize_act(F.f64_to_bf16_bits(rows))
    assert np.isnan(s[0]) and np.isnan(s[3])
    assert s[1] == np.inf and s[2] == np.inf
    assert np.all(q[:4] == 0)
    assert s[4] == 1.0 and q[4].tolist() == [127, 1, -2, 0]
    b = np.array([[1, -2, 3, 4], [5, 6, -7, 8]], np.int8)
    out, _ = R.int8_epilogue(R.int8_accumulate(q, b), s, np.array([0.5, 0.25], np.float32))
    assert np.all(np.isnan(out[:4])) and np.all(np.isfinite(out[4]))


def test_int8_accumulate_brute_force():
    r = np.random.default_rng(21)
    for (m, n, k) in ((3, 4, 5), (2, 3, 200), (1, 1, 1)):
        a = r.integers(-127, 128, size=(m, k)).astype(np.int8)
        b = r.integers(-127, 128, size=(n, k)).astype(np.int8)
        acc = R.int8_accumulate(a, b)
        for i in range(m):
            for j in range(n):
                assert acc[i, j] == sum(int(a[i, t]) * int(b[j, t]) for t in range(k))
    a = np.full((1, 3072), 127, np.int8)
    assert R.int8_accumulate(a, -a)[0, 0] == -3072 * 127 * 127


def test_int8_gemm_golden():
    g = _load("int8_example.json")["gemm"]
    a = np.array(g["a"], np.int8)
    b = np.array(g["b"], np.int8)
    acc = R.int8_accumulate(a, b)
    assert acc.tolist() == g["acc"]
    bias = np.array([int(v, 16) for v in g["bias_bits"]], np.uint16)
    out, tau = R.int8_epilogue(acc, np.array(g["a_scale"], np.float32), np.array(g["b_scale"], np.float32), bias)
    assert np.array_equal(out, np.array(g["out"], float))
    assert np.array_equal(F.f64_to_bf16_bits(out), _hex_array(g["out_bf16_bits"], np.uint16))
    nob, _ = R.int8_epilogue(acc, np.array(g["a_scale"], np.float32), np.array(g["b_scale"], np.float32))
    assert np.array_equal(nob, out - np.array([1.0, -3.0])[None, :])
    assert np.all(tau > 0)


# ------------------------------------------------------------------ FP8 W8A8 (fp8 activations)

def test_fp8_quantize_golden():
    g = _load("fp8_quant_example.json")
    x = synth.bf16_bits_from_f32(np.array([float(v) for v in g["x_values"]], np.float32))[None, :]
    got = R.fp8_quantize_act(x, float(g["input_scale"]))[0]
    assert [f"0x{c:02X}" for c in got] == g["codes"]


def test_e4m3_encoder_round_trips_and_matches_torch():
    """Every finite code decodes and re-encodes to itself; on a dense grid and
    at every midpoint between neighbouring codes (the ties) the encoder agrees
    with torch's float8_e4m3fn cast, an independent round-to-nearest-even."""
    codes = np.arange(256, dtype=np.uint8)
    vals = F.e4m3_to_f64(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(F.f64_to_e4m3_codes(vals[fin]), codes[fin])
    pos = np.unique(vals[fin & (vals >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2
    grid = np.concatenate([np.linspace(-448, 448, 20001), np.linspace(-0.02, 0.02, 20001), mids, -mids])
    grid = grid.astype(np.float32).astype(np.float64)
    want = torch.from_numpy(grid.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.f64_to_e4m3_codes(grid), want)
    assert F.f64_to_e4m3_codes(np.array([449.0, 1e30, -464.0]))[0] == 0x7E      # saturation
    assert list(F.f64_to_e4m3_codes(np.array([1e30, -464.0]))) == [0x7E, 0xFE]


def test_fp8_quantize_error_bound():
    """|dec(q) * s - x| is at most half an E4M3 spacing of x / s (relative 2^-4
    for normals, 2^-10 absolute below 2^-6), or the saturation excess."""
    x = synth.bf16_activation((80,), 16, 512, outlier_p=0.02, outlier_mul=50.0)
    s = 0.01
    q = R.fp8_quantize_act(x, s)
    xv = F.bf16_bits_to_f64(x)
    v = np.clip(xv / s, -448, 448)
    d = F.e4m3_to_f64(q)
    spacing = np.where(np.abs(v) >= 2.0 ** -6, np.ldexp(1.0, np.frexp(np.abs(v))[1] - 1 - 3), 2.0 ** -9)
    assert np.all(np.abs(d - v) <= spacing / 2 * (1 + 1e-6) + 1e-12)
    assert np.any(np.abs(xv / s) > 448)                         # the outliers saturate


@pytest.mark.parametrize("m,n,k", [(1, 3, 5), (3, 4, 64), (2, 2, 130)])
def test_fp8_w8a8_linear_fraction_brute_force(m, n, k):
    r = np.random.default_rng(m * 31 + k)
    xq = r.integers(0, 256, size=(m, k), dtype=np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x38
    w = r.integers(0, 256, size=(n, k), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38
    got, bound = R.fp8_w8a8_linear(xq, w, 0.375)
    xd, wd = F.e4m3_to_f64(xq), F.e4m3_to_f64(w)
    exact = _fraction_linear(wd, xd)
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(float(got[i, j])) - Fraction(3, 8) * exact[i][j]) <= \
                Fraction(2.0 ** -40) * Fraction(float(bound[i, j]) + 1)


def test_fp8_w8a8_equals_w8a16_on_decoded_activation():
    """Every E4M3 value is a bfloat16, so the W8A8 product equals the W8A16
    product of the decoded activation."""
    r = np.random.default_rng(81)
    xq = r.integers(0, 0x7E, size=(5, 96), dtype=np.uint8)
    w = r.integers(0, 0x7E, size=(7, 96), dtype=np.uint8)
    a, _ = R.fp8_w8a8_linear(xq, w, 2.0)
    b, _ = R.fp8_linear(w, F.f64_to_bf16_bits(F.e4m3_to_f64(xq)), 2.0)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ dense bf16 control

def _torch_bf16_values(bits):
    """bfloat16 bits -> float64 through torch's own bfloat16 type (not the
    oracle's decoder)."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


@pytest.mark.parametrize("m,n,k", [(1, 3, 5), (2, 5, 7), (4, 3, 40), (3, 1, 2)])
def test_bf16_linear_fraction_brute_force(m, n, k):
    r = np.random.default_rng(m * 7 + n * 3 + k)
    w = synth.bf16_bits_from_f32((r.standard_normal((n, k)) * 0.05).astype(np.float32))
    x = synth.bf16_bits_from_f32(r.standard_normal((m, k)).astype(np.float32))
    got, bound = R.bf16_linear(w, x, 0.75)
    exact = _fraction_linear(_torch_bf16_values(w), _torch_bf16_values(x))
    for i in range(m):
        for j in range(n):
            assert abs(Fraction(float(got[i, j])) - Fraction(3, 4) * exact[i][j]) <= \
                Fraction(2.0 ** -40) * Fraction(float(bound[i, j]) + 1)
            b = sum(abs(Fraction(float(a)) * Fraction(float(c)))
                    for a, c in zip(_torch_bf16_values(x)[i], _torch_bf16_values(w)[j]))
            assert abs(Fraction(float(bound[i, j])) - Fraction(3, 4) * b) <= Fraction(2.0 ** -40) * (b + 1)


def test_bf16_linear_identity_weight():
    """W = I returns the activation itself (x @ I^T = x), exactly."""
    x = synth.bf16_activation((81,), 3, 24)
    eye = np.where(np.eye(24, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    got, _ = R.bf16_linear(eye, x)
    assert np.array_equal(got, _torch_bf16_values(x))


def test_bf16_linear_equals_fp8_linear_on_widened_weight():
    """Every E4M3 value is a bfloat16: the dense product of the weight widened
    by torch's float8 -> bfloat16 cast equals the W8A16 product."""
    r = np.random.default_rng(82)
    w = r.integers(0, 256, size=(9, 80), dtype=np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x38
    wb = torch.from_numpy(w).view(torch.float8_e4m3fn).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    x = synth.bf16_activation((82,), 4, 80)
    a, ba = R.bf16_linear(wb, x, 1.5)
    b, bb = R.fp8_linear(w, x, 1.5)
    assert np.array_equal(a, b) and np.array_equal(ba, bb)


# ------------------------------------------------------------------ fused epilogue

def test_epilogue_golden():
    g = _load("epilogue_example.json")
    bias = np.array([int(b, 16) for b in g["bias_bits"]], dtype=np.uint16)
    assert np.array_equal(F.bf16_bits_to_f64(bias), np.array(g["bias_values"]))
    out, parts = R.apply_epilogue(np.array(g["value"]), g["row_scale"], g["col_scale"], bias, "relu",
                                  np.array(g["residual"]))
    assert np.array_equal(parts["scaled"], np.array(g["after_scales"]))
    assert np.array_equal(parts["pre"], np.array(g["after_bias"]))
    assert np.array_equal(parts["post"], np.array(g["after_relu"]))
    assert np.array_equal(out, np.array(g["out"]))


def test_epilogue_without_steps_is_identity():
    v = np.random.default_rng(90).standard_normal((3, 5))
    out, parts = R.apply_epilogue(v)
    assert np.array_equal(out, v) and np.array_equal(parts["scale"], np.ones((3, 5)))


@pytest.mark.parametrize("name,fn", [
    ("relu", lambda t: torch.relu(t)),
    ("silu", lambda t: torch.nn.functional.silu(t)),
    ("gelu_tanh", lambda t: torch.nn.functional.gelu(t, approximate="tanh")),
])
def test_activations_match_torch(name, fn):
    v = np.concatenate([np.linspace(-12, 12, 2401), [-80.0, -30.0, 0.0, 30.0, 80.0]])
    want = fn(torch.from_numpy(v)).numpy()
    got = R.activation(v, name)
    # absolute in |v|: where the factor 1 + tanh(.) cancels (large negative v)
    # the two float64 evaluations agree only to a few ulps of v, not of the result
    assert np.all(np.abs(got - want) <= 1e-14 * (1 + np.abs(v)))


def _decimal_activation(v, name):
    """SiLU / tanh-form GELU from their literal definitions in 400-digit
    decimal arithmetic (tanh through exp; enough digits that 1 + tanh(u)
    keeps 40 of them down to v = -20), rounded to float64 at the end."""
    import decimal
    with decimal.localcontext() as ctx:
        ctx.prec = 400
        D = decimal.Decimal
        d = D(repr(float(v)))
        if name == "silu":
            return float(d / (1 + (-d).exp()))
        pi = D("3.14159265358979323846264338327950288419716939937510582097494459230781640628620899")
        u = (2 / pi).sqrt() * (d + D("0.044715") * d * d * d)
        e2 = (2 * u).exp()
        return float(D("0.5") * d * (1 + (e2 - 1) / (e2 + 1)))


@pytest.mark.parametrize("name", ["silu", "gelu_tanh"])
def test_activations_match_high_precision_definition(name):
    """Relative agreement with the literal definition evaluated in 60 digits,
    over the whole range that bfloat16 outputs can hold, tails included
    (for the GELU the float64 literal form would give 0 below v = -6)."""
    v = np.concatenate([np.linspace(-9, 9, 181), [-12.5, -11.0, -10.25, -7.25, 25.0]])
    if name == "silu":
        v = np.concatenate([v, [-95.0, -80.0, -60.0]])
    got = R.activation(v, name)
    want = np.array([_decimal_activation(t, name) for t in v])
    assert np.all(np.abs(got - want) <= 1e-13 * np.abs(want)), np.max(np.abs(got - want) / np.abs(want))
    if name == "gelu_tanh":      # far tail: far below the smallest bfloat16 (2^-133), as defined
        tail = R.activation(np.array([-20.0, -40.0, -1e3]), name)
        assert np.all(np.abs(tail) < 1e-200) and np.all(tail <= 0)


@pytest.mark.parametrize("name", ["silu", "gelu_tanh"])
def test_activation_odd_part_is_identity(name):
    """f(v) - f(-v) = v for SiLU and the tanh-form GELU (both are v times a
    sigmoid-shaped factor g with g(v) + g(-v) = 1): fails on a wrong sign."""
    v = np.linspace(-6, 6, 241)
    assert np.allclose(R.activation(v, name) - R.activation(-v, name), v, rtol=0, atol=1e-12)


def test_grouped_expert_scale_scales_each_experts_rows():
    """The per-expert scale multiplies exactly the rows of that expert's
    groups (inactive groups stay zero, uncovered rows untouched)."""
    r = np.random.default_rng(91)
    w = r.integers(0, 0x7E, size=(3, 6, 40), dtype=np.uint8)
    x = synth.bf16_activation((91,), 12, 40)
    offs = np.array([0, 3, 7, 7, 10])
    ids = np.array([2, -1, 0, 1])
    scale = np.array([0.5, 3.0, -2.0], np.float32)
    raw, braw, wr = R.fp8_grouped(w, x, offs, ids)
    got, bgot, wg = R.fp8_grouped(w, x, offs, ids, scale)
    assert np.array_equal(wr, wg)
    per_row = np.full(12, np.nan)
    per_row[0:3], per_row[3:7], per_row[7:10] = -2.0, 1.0, 3.0   # experts 2, inactive, (empty), 1
    rows = wr
    assert np.array_equal(got[rows], raw[rows] * per_row[rows, None])
    assert np.array_equal(bgot[rows], braw[rows] * np.abs(per_row[rows, None]))
    assert np.all(got[3:7] == 0)


def test_int8_grouped_python_integer_brute_force():
    """Exact Python-integer accumulators per group and expert, the epilogue of
    each row with its own a_scale and its expert's b_scale / bias, zeros for
    an inactive group, untouched rows for uncovered ones."""
    r = np.random.default_rng(92)
    e, n, k, t = 3, 5, 33, 11
    a = r.integers(-127, 128, size=(t, k), dtype=np.int8)
    b = r.integers(-127, 128, size=(e, n, k), dtype=np.int8)
    a_s = r.uniform(0.001, 0.1, t).astype(np.float32)
    b_s = r.uniform(0.001, 0.1, (e, n)).astype(np.float32)
    bias = synth.bf16_bits_from_f32(r.standard_normal((e, n)).astype(np.float32))
    offs = np.array([1, 4, 4, 6, 10])          # row 0 and row 10 uncovered; group 1 empty
    ids = np.array([2, 0, -1, 1])
    acc, _, w_raw = R.int8_grouped(a, b, a_s, b_s, bias, offs, ids, raw=True)
    ref, tau, written = R.int8_grouped(a, b, a_s, b_s, bias, offs, ids)
    assert np.array_equal(w_raw, written)
    assert list(np.flatnonzero(~written)) == [0, 10]
    expert_of_row = {1: 2, 2: 2, 3: 2, 4: -1, 5: -1, 6: 1, 7: 1, 8: 1, 9: 1}
    bias_v = F.bf16_bits_to_f64(bias)
    for row, ex in expert_of_row.items():
        for col in range(n):
            if ex < 0:
                assert acc[row, col] == 0 and ref[row, col] == 0 and tau[row, col] == 0
                continue
            want = sum(int(a[row, i]) * int(b[ex, col, i]) for i in range(k))
            assert acc[row, col] == want
            exact = Fraction(want) * Fraction(float(a_s[row])) * Fraction(float(b_s[ex, col])) + \
                Fraction(float(bias_v[ex, col]))
            assert abs(Fraction(float(ref[row, col])) - exact) <= Fraction(2.0 ** -40) * (abs(exact) + 1)
