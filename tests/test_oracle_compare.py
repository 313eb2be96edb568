"""Pins of the acceptance rules (oracle.compare): they accept what they must
and reject plausible mistakes."""

import numpy as np
import pytest

from oracle import compare as C
from oracle import formats as F


def test_bf16_ordered_and_ulp():
    b = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3F80, 0x3F81, 0x7F7F], np.uint16)
    o = C.bf16_ordered(b)
    assert o[0] == o[1] == 0 and o[2] == 1 and o[3] == -1 and o[5] - o[4] == 1
    u = C.bf16_ulp(np.array([0x3F80, 0x4000, 0x0000, 0x0080], np.uint16))
    assert list(u) == [2.0 ** -7, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133]


def test_check_bf16_accepts_neighbours_rejects_two_ulps():
    ref = np.array([1.0 + 2.0 ** -9, 3.0, -5.25, 0.0])
    r = F.f64_to_bf16_bits(ref)
    tau = np.zeros(4)
    assert C.check_bf16(r, ref, tau)
    def step(bits, d):
        # move d places along the ordered bf16 line
        o = C.bf16_ordered(bits) + d
        return np.where(o < 0, 0x8000 | (-o), o).astype(np.uint16)
    assert C.check_bf16(step(r, 1), ref, tau)
    assert C.check_bf16(step(r, -1), ref, tau)
    assert not C.check_bf16(step(r, -2), ref, tau)
    bad = r.copy()
    bad[1] += 2
    res = C.check_bf16(bad, ref, tau)
    assert not res and res.n_bad == 1
    # +0 vs -0 are equal
    assert C.check_bf16(np.array([0x8000], np.uint16), np.array([0.0]), np.zeros(1))


def test_check_bf16_clause2_cancellation():
    ref = np.array([1e-6])
    gpu = F.f64_to_bf16_bits(np.array([3e-6]))      # many bf16 ulps away but within tau
    assert C.check_bf16(gpu, ref, np.array([5e-6])).n_clause2 == 1
    assert not C.check_bf16(gpu, ref, np.array([1e-7]))


def test_check_f32_bound_and_nan():
    ref = np.array([1.0, 2.0, np.nan])
    b = np.array([100.0, 100.0, 1.0])
    assert C.check_f32(np.array([1.1, 1.9, np.nan], np.float32), ref, b)
    assert not C.check_f32(np.array([1.3, 2.0, np.nan], np.float32), ref, b)
    assert not C.check_f32(np.array([1.0, 2.0, 0.0], np.float32), ref, b)
    assert not C.check_f32(np.array([np.nan, 2.0, np.nan], np.float32), ref, b)


def test_tolerance_rejects_a_dropped_row_of_terms():
    """A kernel that drops every product of one K-chunk (1/16 of the terms)
    must fail the rule on realistic data."""
    r = np.random.default_rng(0)
    k = 4096
    x = r.standard_normal((1, k))
    w = r.standard_normal((64, k)) * 0.02
    ref = x @ w.T
    bound = np.abs(x) @ np.abs(w).T
    mask = np.ones(k)
    mask[:256] = 0
    bad = (x * mask) @ w.T
    assert not C.check_f32(bad.astype(np.float32), ref, bound)


# ------------------------------------------------------------------ fused-epilogue tolerance

import functools  # noqa: E402

import synth  # noqa: E402
from oracle import ref as R  # noqa: E402


def _f32_activation(v, act):
    """The activation evaluated in float32 as x sigmoid(z) (SiLU: z = v; tanh
    GELU: 0.5 v (1 + tanh(u)) = v sigmoid(2u)), each step rounded to float32,
    exp correctly rounded, and the sigmoid taken from exp(-|z|) so that
    nothing overflows or cancels."""
    f = np.float32
    v = v.astype(np.float32)
    if act == "none":
        return v
    if act == "relu":
        return np.maximum(v, f(0))
    z = v if act == "silu" else (f(2) * (f(0.7978845608028654) * (v + f(0.044715) * v * v * v))).astype(np.float32)
    e = np.exp(-np.abs(z).astype(np.float64)).astype(np.float32)
    d = (f(1) + e).astype(np.float32)
    return np.where(z >= 0, v / d, (v * e).astype(np.float32) / d).astype(np.float32)


def _f32_epilogue(acc32, alpha, row, col, bias_bits, act, residual, *, bias_first=False, act_fn=None,
                  scales_after_act=False):
    """The fused epilogue evaluated step by step in float32, as a kernel
    does; the keyword switches plant the plausible mistakes."""
    v = acc32 * np.float32(alpha)
    bias = None if bias_bits is None else F.bf16_bits_to_f64(bias_bits).astype(np.float32)[None, :]
    if bias_first and bias is not None:
        v = v + bias
    if not scales_after_act:
        if row is not None:
            v = v * row[:, None]
        if col is not None:
            v = v * col[None, :]
    if not bias_first and bias is not None:
        v = v + bias
    v = (act_fn or _f32_activation)(v, act)
    if scales_after_act:
        if row is not None:
            v = v * row[:, None]
        if col is not None:
            v = v * col[None, :]
    if residual is not None:
        v = v + residual
    return v.astype(np.float32)


def _gelu_erf(v, act):
    from scipy.special import erf
    v = v.astype(np.float64)
    return (0.5 * v * (1.0 + erf(v / np.sqrt(2.0)))).astype(np.float32)


def _silu_sign_error(v, act):
    v = v.astype(np.float64)
    with np.errstate(over="ignore"):
        return (v / (1.0 + np.exp(v))).astype(np.float32)


def _sloppy_exp_silu(v, act):
    """SiLU through an exponential with 1e-4 relative error (a short series)."""
    v = v.astype(np.float64)
    with np.errstate(over="ignore"):
        return (v / (1.0 + np.exp(-v) * (1.0 + 1e-4))).astype(np.float32)


def _bf16_exp_silu(v, act):
    """SiLU through an exponential rounded to bfloat16 (8 significant bits)."""
    v = v.astype(np.float64)
    with np.errstate(over="ignore"):
        e = F.bf16_bits_to_f64(F.f64_to_bf16_bits(np.exp(-v)))
        return (v / (1.0 + e)).astype(np.float32)


@functools.lru_cache(maxsize=None)
def _realistic(m=16, n=512, k=4096):
    """W8A16 at a decode K: E4M3 codes of N(0, 0.02^2) with their per-tensor
    scale, bf16 N(0, 1) activation; the raw fp64 reference and bound, a float32
    product (BLAS order) and the scale (the alpha that gives the layer's real
    output magnitude, about N(0, 1.3^2))."""
    w, s = synth.fp8_weight((400,), n, k)
    xb = synth.bf16_activation((401,), m, k)
    raw, bound = R.fp8_linear(w, xb, 1.0)
    acc32 = F.bf16_bits_to_f64(xb).astype(np.float32) @ F.e4m3_to_f64(w).astype(np.float32).T
    return raw, bound, acc32.astype(np.float32), float(s)


@functools.lru_cache(maxsize=None)
def _exact(m=16, n=512, k=512):
    """Dyadic W8A16 (every float32 partial sum exact): the raw product is
    exact in float32 in any order."""
    w = synth.dyadic_fp8_weight((402,), n, k)
    xb = synth.dyadic_activation((403,), m, k)
    raw, bound = R.fp8_linear(w, xb, 1.0)
    acc32 = raw.astype(np.float32)
    assert np.array_equal(acc32.astype(np.float64), raw)
    return raw, bound, acc32


def _epilogue_inputs(raw, seed, integer=False):
    m, n = raw.shape
    r = np.random.default_rng(seed)
    typical = float(np.median(np.abs(raw)))
    if integer:
        row = np.ldexp(1.0, r.integers(-2, 1, m)).astype(np.float32)
        col = (np.ldexp(1.0, r.integers(-1, 1, n)) * r.choice([-1, 1], n)).astype(np.float32)
        bias = synth.bf16_bits_from_f32(r.integers(-8, 9, n).astype(np.float32))
        res = r.integers(-50, 51, (m, n)).astype(np.float32)
    else:
        row = r.uniform(0.5, 2.0, m).astype(np.float32)
        col = r.uniform(-2.0, 2.0, n).astype(np.float32)
        bias = synth.bf16_bits_from_f32(r.standard_normal(n).astype(np.float32))
        res = (r.standard_normal((m, n)) * typical).astype(np.float32)
    return row, col, bias, res


@pytest.mark.parametrize("act", ["none", "relu", "silu", "gelu_tanh"])
def test_epilogue_tolerance_accepts_float32_evaluation(act):
    """A correct float32 evaluation of the fused epilogue, on a float32
    matmul (realistic data) or on an exact one (dyadic data, tolerance
    without the matmul term), is accepted."""
    for data, exact in ((_realistic(), False), (_exact(), True)):
        raw, bound, acc32 = data[:3]
        alpha = data[3] if not exact else 0.75
        row, col, bias, res = _epilogue_inputs(raw * alpha, 7, integer=exact)
        ref, parts = R.apply_epilogue(raw * alpha, row, col, bias, act, res)
        tau = C.epilogue_tolerance(alpha * bound, parts, act, matmul_exact=exact)
        got = _f32_epilogue(acc32, alpha, row, col, bias, act, res)
        assert C.check_f32_tau(got, ref, tau), (act, exact)


MISTAKES = [  # (name, activation, keyword switches of _f32_epilogue)
    ("bias before the scales", "silu", dict(bias_first=True)),
    ("scales after the activation", "gelu_tanh", dict(scales_after_act=True)),
    ("SiLU sign error", "silu", dict(act_fn=_silu_sign_error)),
    ("dropped residual", "none", dict(drop_residual=True)),
]


@pytest.mark.parametrize("name,act,kw", MISTAKES, ids=[m[0] for m in MISTAKES])
def test_epilogue_tolerance_rejects_mistakes_at_workload_magnitude(name, act, kw):
    """On realistic data (where the matmul term of the tolerance is large)
    a wrong step order, a sign error or a dropped step still fails."""
    raw, bound, acc32, alpha = _realistic()
    row, col, bias, res = _epilogue_inputs(raw * alpha, 8)
    ref, parts = R.apply_epilogue(raw * alpha, row, col, bias, act, res)
    tau = C.epilogue_tolerance(alpha * bound, parts, act)
    kw = dict(kw)
    residual = None if kw.pop("drop_residual", False) else res
    got = _f32_epilogue(acc32, alpha, row, col, bias, act, residual, **kw)
    assert not C.check_f32_tau(got, ref, tau), name


@pytest.mark.parametrize("name,act,fn", [("erf-form GELU for the tanh form", "gelu_tanh", _gelu_erf),
                                         ("exp with 1e-4 relative error", "silu", _sloppy_exp_silu)])
def test_exact_matmul_tolerance_rejects_activation_mistakes(name, act, fn):
    """With an exact matmul the tolerance keeps only the activation's own
    float32 slack: an erf-form GELU in place of the tanh form, or an
    exponential good to only 1e-4, fails (at workload magnitudes the matmul
    term would hide both)."""
    raw, bound, acc32 = _exact()
    row, col, bias, res = _epilogue_inputs(raw, 9, integer=True)
    ref, parts = R.apply_epilogue(raw, row, col, bias, act, res)
    tau = C.epilogue_tolerance(bound, parts, act, matmul_exact=True)
    assert not C.check_f32_tau(_f32_epilogue(acc32, 1.0, row, col, bias, act, res, act_fn=fn), ref, tau), name
    loose = C.epilogue_tolerance(bound, parts, act)
    assert C.check_f32_tau(_f32_epilogue(acc32, 1.0, row, col, bias, act, res, act_fn=fn), ref, loose), \
        "the matmul term alone would have hidden this mistake"


# ------------------------------------------------------------------ clause-2 shares

@functools.lru_cache(maxsize=None)
def _sequential_f32(m=64, n=1024, k=4096):
    """Realistic W8A16 summed in plain sequential float32 (the least
    accurate order a correct kernel could take)."""
    w, _ = synth.fp8_weight((404,), n, k)
    xb = synth.bf16_activation((405,), m, k)
    raw, bound = R.fp8_linear(w, xb, 1.0)
    wd = F.e4m3_to_f64(w).astype(np.float32)
    xd = F.bf16_bits_to_f64(xb).astype(np.float32)
    acc = np.zeros((m, n), np.float32)
    for kk in range(k):
        acc += np.outer(xd[:, kk], wd[:, kk]).astype(np.float32)
    return raw, bound, acc, xd, wd


def test_clause2_share_f32_covers_sequential_float32_sums():
    """Sequential float32 summation stays inside the float32 share; an
    accumulator that keeps only bfloat16 precision (each 32-product partial
    sum rounded to bf16) needs clause 2 far more often and exceeds it."""
    raw, bound, acc, xd, wd = _sequential_f32()
    tau = C.fp_tolerance(bound)
    res = C.check_bf16(F.f64_to_bf16_bits(acc.astype(np.float64)), raw, tau)
    assert res and res.n_clause2 <= C.clause2_budget(raw), res
    bad = np.zeros_like(acc)
    for j in range(xd.shape[1] // 32):
        sl = slice(32 * j, 32 * j + 32)
        bad = (bad + (xd[:, sl] @ wd[:, sl].T).astype(np.float32)).astype(np.float32)
        bad = F.bf16_bits_to_f64(F.f64_to_bf16_bits(bad.astype(np.float64))).astype(np.float32)
    res_bad = C.check_bf16(F.f64_to_bf16_bits(bad.astype(np.float64)), raw, tau)
    assert not res_bad or res_bad.n_clause2 > C.clause2_budget(raw), res_bad


def _gelu_sigmoid_approx(v, act):
    """The other common GELU approximation, v sigmoid(1.702 v), in place of
    the tanh form (within 0.02 of it everywhere)."""
    v = v.astype(np.float64)
    with np.errstate(over="ignore"):
        return (v / (1.0 + np.exp(-1.702 * v))).astype(np.float32)


def test_clause2_share_epilogue_covers_float32_activations():
    """The fused epilogue (bias, SiLU or tanh GELU) evaluated in float32 on the
    sequential float32 sum, at a real layer's output magnitude: within the
    epilogue share.  The sigmoid approximation of the GELU in place of the
    tanh form is rejected (by the tolerance where the column scale is small,
    by the share elsewhere)."""
    raw, bound, acc, _, _ = _sequential_f32()
    alpha = float(synth.fp8_weight((404,), 1024, 4096)[1])
    r = np.random.default_rng(10)
    bias = synth.bf16_bits_from_f32(r.standard_normal(raw.shape[1]).astype(np.float32))
    col = r.uniform(-2.0, 2.0, raw.shape[1]).astype(np.float32)
    for act in ("silu", "gelu_tanh"):
        ref, parts = R.apply_epilogue(raw * alpha, None, col, bias, act, None)
        tau = C.epilogue_tolerance(alpha * bound, parts, act)
        got = _f32_epilogue(acc, alpha, None, col, bias, act, None)
        res = C.check_bf16(F.f64_to_bf16_bits(got.astype(np.float64)), ref, tau)
        assert res and res.n_clause2 <= C.clause2_budget(ref, C.CLAUSE2_SHARE_EPILOGUE), (act, res)
    ref, parts = R.apply_epilogue(raw * alpha, None, col, bias, "gelu_tanh", None)
    tau = C.epilogue_tolerance(alpha * bound, parts, "gelu_tanh")
    got = _f32_epilogue(acc, alpha, None, col, bias, "gelu_tanh", None, act_fn=_gelu_sigmoid_approx)
    res = C.check_bf16(F.f64_to_bf16_bits(got.astype(np.float64)), ref, tau)
    assert not res or res.n_clause2 > C.clause2_budget(ref, C.CLAUSE2_SHARE_EPILOGUE), res


def _block_rounded_w8a8(xd, wd, bits):
    """W8A8 product whose 64-product blocks are each rounded to a grid
    2^-bits below the block's sum of magnitudes, then added in float32."""
    acc = np.zeros((xd.shape[0], wd.shape[0]), np.float32)
    for j in range(xd.shape[1] // 64):
        sl = slice(64 * j, 64 * j + 64)
        s = xd[:, sl] @ wd[:, sl].T
        b = np.abs(xd[:, sl]) @ np.abs(wd[:, sl]).T
        step = np.ldexp(1.0, (np.floor(np.log2(np.maximum(b, 1e-300))) - bits).astype(np.int64))
        acc = (acc + (np.rint(s / step) * step).astype(np.float32)).astype(np.float32)
    return acc


def test_clause2_share_f8f6f4_covers_the_measured_accumulation():
    """The fp8 matrix instruction's accumulation, modelled as 64-product
    blocks rounded 14 bits below their sum of magnitudes (this reproduces the
    measured clause-2 rate of about 0.3 % and an error near 1e-5 B), stays
    within the W8A8 share with margin; four times coarser blocks (12 bits)
    exceed it."""
    c = synth.fp8_w8a8_case(3072)
    q = R.fp8_quantize_act(c.x[:96], c.input_scale)
    xd, wd = F.e4m3_to_f64(q), F.e4m3_to_f64(c.w[:1024])
    ref, bound = xd @ wd.T, np.abs(xd) @ np.abs(wd).T
    tau = C.fp_tolerance(bound)
    budget = C.clause2_budget(ref, C.CLAUSE2_SHARE_F8F6F4)
    res = C.check_bf16(F.f64_to_bf16_bits(_block_rounded_w8a8(xd, wd, 14).astype(np.float64)), ref, tau)
    assert res and 3 * res.n_clause2 <= budget, res
    res = C.check_bf16(F.f64_to_bf16_bits(_block_rounded_w8a8(xd, wd, 12).astype(np.float64)), ref, tau)
    assert not res or res.n_clause2 > budget, res
