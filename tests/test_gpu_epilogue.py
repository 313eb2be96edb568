"""GPU parity of the fused epilogues (qlinear_*_gemm_epilogue) and of the
per-expert scale of the grouped calls (qlinear_*_grouped_gemm_scaled) against
the CPU oracle, through the C ABI, on every kernel family."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import compare as C
from oracle import formats as F
from oracle import ref as R
from gpu_util import DEV, bf16_bits, show, to_dev, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import weight_quantized_linear_amd as q
    return q


# (name, kind, path, M, N, K): every kernel that stores an fp8 / NVFP4 / bf16 output
FAMILIES = [
    ("fp8 gemv", "fp8", "gemv", 3, 500, 4096),
    ("fp8 gemv any-K", "fp8", "gemv", 1, 257, 1000),
    ("fp8 skinny 16x16x32", "fp8", "skinny", 9, 1000, 4096),
    ("fp8 skinny activation-in-LDS", "fp8", "skinny", 4, 5000, 4096),
    ("fp8 skinny 4x4x4", "fp8", "skinny", 2, 700, 1040),
    ("fp8 skinny LDS wide-N", "fp8", "skinny", 12, 66000, 192),
    ("fp8 streaming split-K", "fp8", "splitk", 12, 1000, 8192),
    ("fp8 skinny split-K", "fp8", "splitk", 12, 1000, 8256),
    ("fp8 tiled split-K", "fp8", "tiled", 20, 1000, 2048),
    ("fp8 tiled whole-K", "fp8", "tiled", 300, 700, 1024),
    ("fp8 tiled 256x256", "fp8", "tiled", 2048, 8200, 64),
    ("fp8 tiled register-staged", "fp8", "tiled", 40, 100, 1000),
    ("nvfp4 gemv", "nvfp4", "auto", 2, 600, 4096),
    ("nvfp4 tiled split-K", "nvfp4", "auto", 64, 4096, 1024),
    ("nvfp4 tiled whole-K", "nvfp4", "auto", 600, 1000, 512),
    ("nvfp4 tiled register-staged", "nvfp4", "auto", 33, 100, 48),
    ("bf16 gemv", "bf16", "auto", 1, 999, 4096),
    ("bf16 skinny", "bf16", "auto", 12, 2000, 1024),
    ("bf16 tiled", "bf16", "auto", 100, 700, 2048),
]

# (name, row scale, column scale, bias, activation, residual): "alias" adds the
# output buffer's own contents
EPILOGUES = [
    ("all+relu", True, True, True, "relu", "bf16"),
    ("silu+f32 residual", False, False, False, "silu", "f32"),
    ("gelu+bias", False, True, True, "gelu_tanh", None),
    ("row scale", True, False, False, "none", None),
    ("residual in place", False, False, True, "none", "alias"),
]


def _weights(kind, key, n, k, dyadic=False):
    """(device args, oracle linear of x_bits and alpha, the weight's own
    per-tensor scale: the alpha that gives a real layer's output magnitude)."""
    if kind == "fp8":
        if dyadic:
            w, s = synth.dyadic_fp8_weight(key, n, k), 1.0
        else:
            w, s = synth.fp8_weight(key, n, k)
        return (to_dev_u8(w),), lambda x, a: R.fp8_linear(w, x, a), float(s)
    if kind == "nvfp4":
        if dyadic:
            (p, sc), g = synth.dyadic_nvfp4_weight(key, n, k), 1.0
        else:
            p, sc, g = synth.nvfp4_weight(key, n, k)
        return (to_dev_u8(p), to_dev_u8(sc)), lambda x, a: R.nvfp4_linear(p, sc, x, a), float(g)
    w = synth.dyadic_bf16_weight(key, n, k) if dyadic else synth.bf16_weight(key, n, k)
    return (to_dev_bf16(w),), lambda x, a: R.bf16_linear(w, x, a), 1.0


def _call(q, kind, path, wargs, x, out, out_dtype, alpha, **epi):
    if kind == "fp8":
        return q.fp8_gemm(wargs[0], x, out=out, out_dtype=out_dtype, alpha=alpha, path=path, **epi)
    if kind == "nvfp4":
        return q.nvfp4_gemm(wargs[0], wargs[1], x, out=out, out_dtype=out_dtype, alpha=alpha, **epi)
    return q.bf16_gemm(wargs[0], x, out=out, out_dtype=out_dtype, alpha=alpha, **epi)


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
@pytest.mark.parametrize("epi", EPILOGUES, ids=[e[0] for e in EPILOGUES])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_epilogue_within_tolerance(q, fam, epi, out_dtype):
    name, kind, path, m, n, k = fam
    ename, use_row, use_col, use_bias, act, res = epi
    key = (60, m, n, k)
    wargs, linear, scale = _weights(kind, key, n, k)
    xb = synth.bf16_activation(key + (1,), m, k)
    r = synth.rng_for(*key, 2)
    alpha = float(np.float32(0.75 * scale))   # a real layer's magnitude: the activations see their curved range
    row = r.uniform(0.5, 2.0, m).astype(np.float32) if use_row else None
    col = r.uniform(-2.0, 2.0, n).astype(np.float32) if use_col else None
    bias = synth.bf16_bits_from_f32(r.standard_normal(n).astype(np.float32)) if use_bias else None
    raw, bound = linear(xb, alpha)
    typical = float(np.median(np.abs(raw))) + 1e-30
    out = torch.empty((m, n), dtype=out_dtype, device=DEV)
    residual_vals = None
    residual = None
    if res == "alias":
        init = (r.standard_normal((m, n)) * typical).astype(np.float32)
        if out_dtype == torch.bfloat16:
            ib = synth.bf16_bits_from_f32(init)
            out.copy_(to_dev_bf16(ib))
            residual_vals = F.bf16_bits_to_f64(ib)
        else:
            out.copy_(torch.from_numpy(init))
            residual_vals = init.astype(np.float64)
        residual = out
    elif res is not None:
        rv = (r.standard_normal((m, n)) * typical).astype(np.float32)
        if res == "bf16":
            rb = synth.bf16_bits_from_f32(rv)
            residual = to_dev_bf16(rb)
            residual_vals = F.bf16_bits_to_f64(rb)
        else:
            residual = torch.from_numpy(rv).to(DEV)
            residual_vals = rv.astype(np.float64)
    ref, parts = R.apply_epilogue(raw, row, col, bias, act, residual_vals)
    tau = C.epilogue_tolerance(bound, parts, act)
    kw = dict(activation=act)
    if row is not None:
        kw["row_scale"] = to_dev(row)
    if col is not None:
        kw["col_scale"] = to_dev(col)
    if bias is not None:
        kw["bias"] = to_dev_bf16(bias)
    if residual is not None:
        kw["residual"] = residual
    show("epilogue", name, ename, out_dtype, m, n, k)
    _call(q, kind, path, wargs, to_dev_bf16(xb), out, out_dtype, alpha, **kw)
    torch.cuda.synchronize()
    if out_dtype == torch.float32:
        res_ = C.check_f32_tau(out.cpu().numpy(), ref, tau)
        assert res_, res_
    else:
        res_ = C.check_bf16(bf16_bits(out), ref, tau)
        assert res_, res_
        assert res_.n_clause2 <= C.clause2_budget(ref, C.CLAUSE2_SHARE_EPILOGUE), res_


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_epilogue_exact_inputs_are_bit_exact(q, fam):
    """Exact inputs, power-of-two scales, integer bias and residual, ReLU:
    every step is exact in float32, so the output is the oracle's exactly."""
    name, kind, path, m, n, k = fam
    key = (61, m, n, k)
    wargs, linear, _ = _weights(kind, key, n, k, dyadic=True)
    xb = synth.dyadic_activation(key + (1,), m, k)
    r = synth.rng_for(*key, 2)
    # scaled values stay multiples of 2^-5 below 2^19 in magnitude: exact in float32
    row = np.ldexp(1.0, r.integers(0, 3, m)).astype(np.float32)
    col = (np.ldexp(1.0, r.integers(-1, 2, n)) * r.choice([-1, 1], n)).astype(np.float32)
    bias = synth.bf16_bits_from_f32(r.integers(-50, 51, n).astype(np.float32))
    resv = r.integers(-100, 101, (m, n)).astype(np.float32)
    raw, _ = linear(xb, 1.0)
    ref, _ = R.apply_epilogue(raw, row, col, bias, "relu", resv)
    for out_dtype in (torch.float32, torch.bfloat16):
        show("epilogue exact", name, out_dtype)
        out = _call(q, kind, path, wargs, to_dev_bf16(xb), None, out_dtype, 1.0, row_scale=to_dev(row),
                    col_scale=to_dev(col), bias=to_dev_bf16(bias), residual=to_dev(resv), activation="relu")
        if out_dtype == torch.float32:
            assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))
        else:
            assert np.array_equal(bf16_bits(out), F.f64_to_bf16_bits(ref))


@pytest.mark.parametrize("fam", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_epilogue_exact_matmul_silu_gelu(q, fam):
    """Exact inputs and power-of-two scales: the value entering the
    activation equals the oracle's, so the tolerance keeps only the float32
    slack of SiLU / tanh GELU themselves (no matmul term).  This checks the
    activations' form and the device exp at their own precision."""
    name, kind, path, m, n, k = fam
    key = (66, m, n, k)
    wargs, linear, _ = _weights(kind, key, n, k, dyadic=True)
    xb = synth.dyadic_activation(key + (1,), m, k)
    r = synth.rng_for(*key, 2)
    raw, bound = linear(xb, 1.0)
    med = float(np.median(np.abs(raw[raw != 0]))) if np.any(raw != 0) else 1.0
    alpha = float(np.ldexp(1.0, -int(np.round(np.log2(med)))))    # power of two: typical |v| near 1
    raw, bound = raw * alpha, bound * alpha
    row = np.ldexp(1.0, r.integers(-1, 2, m)).astype(np.float32)
    col = (np.ldexp(1.0, r.integers(-1, 1, n)) * r.choice([-1, 1], n)).astype(np.float32)
    bias = synth.bf16_bits_from_f32((r.integers(-12, 13, n) / 4).astype(np.float32))
    resv = r.integers(-20, 21, (m, n)).astype(np.float32)
    for act in ("silu", "gelu_tanh"):
        ref, parts = R.apply_epilogue(raw, row, col, bias, act, resv)
        tau = C.epilogue_tolerance(bound, parts, act, matmul_exact=True)
        for out_dtype in (torch.float32, torch.bfloat16):
            show("epilogue exact matmul", name, act, out_dtype)
            out = _call(q, kind, path, wargs, to_dev_bf16(xb), None, out_dtype, alpha, row_scale=to_dev(row),
                        col_scale=to_dev(col), bias=to_dev_bf16(bias), residual=to_dev(resv), activation=act)
            if out_dtype == torch.float32:
                res_ = C.check_f32_tau(out.cpu().numpy(), ref, tau)
            else:
                res_ = C.check_bf16(bf16_bits(out), ref, tau)
                assert res_.n_clause2 <= C.clause2_budget(ref), res_
            assert res_, (act, res_)


def test_empty_epilogue_is_the_plain_call(q):
    wc, _ = synth.fp8_weight((62,), 800, 1024)
    xb = synth.bf16_activation((62, 1), 40, 1024)
    w, x = to_dev_u8(wc), to_dev_bf16(xb)
    show("epilogue empty descriptor")
    plain = q.fp8_gemm(w, x, out_dtype=torch.float32, workspace=None)   # no workspace, like the C call below
    d = q.EpilogueDesc(None, None, None, None, 0, 0, 0)
    out = torch.empty_like(plain)
    st = q.lib.qlinear_fp8_gemm_epilogue(ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(x.data_ptr()),
                                         ctypes.c_void_p(out.data_ptr()), 0, 40, 800, 1024, 1.0, ctypes.byref(d),
                                         None)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(out, plain)


def test_epilogue_rejects_bad_descriptors(q):
    w = torch.zeros((64, 128), dtype=torch.uint8, device=DEV)
    x = torch.zeros((4, 128), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((4, 64), dtype=torch.float32, device=DEV)
    res = torch.zeros((4, 64), dtype=torch.float32, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    show("epilogue bad descriptors")
    bad = [
        q.EpilogueDesc(None, None, None, None, 0, 0, 7),                         # unknown activation
        q.EpilogueDesc(None, None, None, res.data_ptr(), 63, 0, 0),              # residual_ld < N
        q.EpilogueDesc(None, None, None, res.data_ptr(), 64, 2, 0),              # residual type int32
        q.EpilogueDesc(res.data_ptr() + 2, None, None, None, 0, 0, 0),           # misaligned row_scale
        q.EpilogueDesc(None, None, res.data_ptr() + 1, None, 0, 0, 0),           # misaligned bias
    ]
    for d in bad:
        st = q.lib.qlinear_fp8_gemm_epilogue(p(w), p(x), p(out), 0, 4, 64, 128, 1.0, ctypes.byref(d), None)
        assert st == q.ERR_INVALID_ARG
    torch.cuda.synchronize()


# ------------------------------------------------------------------ grouped: per-expert scale

def _ids_offs():
    offs = np.array([0, 1, 129, 129, 300, 401])
    ids = np.array([4, 0, 1, -1, 2], np.int32)
    return offs, ids


@pytest.mark.parametrize("kind,k", [("fp8", 1024), ("fp8", 1000), ("nvfp4", 1024), ("nvfp4", 1040)])
def test_grouped_expert_scale_bit_exact(q, kind, k):
    e, n, t = 5, 130, 401
    offs, ids = _ids_offs()
    scale = np.array([0.5, -2.0, 4.0, 1.0, 0.25], np.float32)
    x = synth.dyadic_activation((63, k), t, k)
    dev_offs = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    dev_ids = torch.from_numpy(ids).to(DEV)
    if kind == "fp8":
        w = synth.dyadic_fp8_weight((64, k), e * n, k).reshape(e, n, k)
        ref, _, written = R.fp8_grouped(w, x, offs, ids, scale)
        call = lambda dt: q.fp8_grouped_gemm(to_dev_u8(w), to_dev_bf16(x), dev_offs, dev_ids,  # noqa: E731
                                             out_dtype=dt, max_tokens_per_group=1, expert_scale=to_dev(scale))
    else:
        p, s = synth.dyadic_nvfp4_weight((64, k), e * n, k)
        p, s = p.reshape(e, n, k // 2), s.reshape(e, n, k // 16)
        ref, _, written = R.nvfp4_grouped(p, s, x, offs, ids, scale)
        call = lambda dt: q.nvfp4_grouped_gemm(to_dev_u8(p), to_dev_u8(s), to_dev_bf16(x), dev_offs,  # noqa: E731
                                               dev_ids, out_dtype=dt, max_tokens_per_group=1,
                                               expert_scale=to_dev(scale))
    assert written.all()
    show("grouped expert scale", kind, k)
    assert np.array_equal(call(torch.float32).cpu().numpy(), ref.astype(np.float32))
    assert np.array_equal(bf16_bits(call(torch.bfloat16)), F.f64_to_bf16_bits(ref))


def test_grouped_expert_scale_workload(q):
    c = synth.config4_case()
    e = c.w.shape[0]
    scale = synth.rng_for(65).uniform(0.001, 0.01, e).astype(np.float32)
    t, n = c.x.shape[0], c.w.shape[1]
    show("grouped expert scale workload", c.name)
    out = q.fp8_grouped_gemm(to_dev_u8(c.w), to_dev_bf16(c.x), torch.from_numpy(c.a_offsets.astype(np.int32)).to(DEV),
                             torch.from_numpy(c.expert_ids.astype(np.int32)).to(DEV), out_dtype=torch.bfloat16,
                             max_tokens_per_group=c.max_tokens, expert_scale=to_dev(scale))
    torch.cuda.synchronize()
    ref, bound, written = R.fp8_grouped(c.w, c.x, c.a_offsets, c.expert_ids, scale)
    got = bf16_bits(out)
    res = C.check_bf16(got[written], ref[written], C.fp_tolerance(bound[written]))
    assert res and res.n_clause2 <= C.clause2_budget(ref[written]), res
