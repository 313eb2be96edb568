"""GPU parity of the grouped MoE W8A8 int8 call (qlinear_int8_grouped_gemm)
against the CPU oracle, through the C ABI.  The activation codes and scales
given to the GPU are the oracle's own quantisation of the seeded activation."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import compare as C
from oracle import ref as R
from gpu_util import DEV, bf16_bits, show, to_dev, to_dev_bf16, to_dev_i8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import weight_quantized_linear_amd as q
    return q


def _call(q, a, b, sa, sb, bias, offs, ids, out=None, out_dtype=torch.bfloat16, max_tokens=None):
    return q.int8_grouped_gemm(to_dev_i8(a), to_dev_i8(b), None if sa is None else to_dev(sa),
                               None if sb is None else to_dev(sb), torch.from_numpy(np.asarray(offs, np.int32)).to(DEV),
                               torch.from_numpy(np.asarray(ids, np.int32)).to(DEV),
                               bias=None if bias is None else to_dev_bf16(bias), out=out, out_dtype=out_dtype,
                               max_tokens_per_group=max_tokens)


@pytest.fixture(scope="module")
def workload():
    c = synth.grouped_int8_case()
    a, sa = R.int8_quantize_act(c.x)
    return c, a, sa


def test_grouped_int8_workload_accumulators_bit_exact(q, workload):
    c, a, sa = workload
    t, n = a.shape[0], c.b.shape[1]
    show("grouped int8 workload raw", c.name)
    out = torch.full((t, n), -7, dtype=torch.int32, device=DEV)
    _call(q, a, c.b, None, None, None, c.a_offsets, c.expert_ids, out=out, out_dtype=torch.int32,
          max_tokens=c.max_tokens)
    torch.cuda.synchronize()
    acc, _, written = R.int8_grouped(a, c.b, sa, c.b_scale, c.bias, c.a_offsets, c.expert_ids, raw=True)
    got = out.cpu().numpy()
    assert np.array_equal(got[written], acc[written].astype(np.int32))
    assert np.all(got[~written] == -7)


def test_grouped_int8_workload_bf16(q, workload):
    c, a, sa = workload
    show("grouped int8 workload bf16", c.name)
    out = _call(q, a, c.b, sa, c.b_scale, c.bias, c.a_offsets, c.expert_ids, max_tokens=c.max_tokens)
    torch.cuda.synchronize()
    ref, tau, written = R.int8_grouped(a, c.b, sa, c.b_scale, c.bias, c.a_offsets, c.expert_ids)
    got = bf16_bits(out)
    res = C.check_bf16(got[written], ref[written], tau[written])
    assert res and res.n_clause2 <= C.clause2_budget(ref[written]), res
    inactive = np.zeros(a.shape[0], bool)
    for z in np.flatnonzero(c.expert_ids == -1):
        inactive[c.a_offsets[z]:c.a_offsets[z + 1]] = True
    assert inactive.sum() == 40 and np.all(got[inactive] == 0)


# K % 128 == 0 (LDS kernel, 128-byte strips), K % 64 == 0 (64-byte strips), K % 16 == 0
# (register-staged, wide loads), neither
@pytest.mark.parametrize("k", [256, 1024, 192, 208, 100])
@pytest.mark.parametrize("with_bias", [True, False])
def test_grouped_int8_ragged_cases(q, k, with_bias):
    e, n, t = 4, 200, 300
    r = np.random.default_rng(k)
    b, sb = synth.int8_weight((74, k), e * n, k)
    b, sb = b.reshape(e, n, k), sb.reshape(e, n)
    bias = synth.bf16_bias((74, k, 1), e * n).reshape(e, n) if with_bias else None
    x = synth.bf16_activation((75, k), t, k, outlier_p=0.01)
    a, sa = R.int8_quantize_act(x)
    # rows 0..9 uncovered; group 1 empty; group 2 inactive; group 3 id past E;
    # group 5 runs past T (clipped); group 6 has end < start (empty).
    offs = np.array([10, 60, 60, 90, 100, 260, 400, 150], np.int64)
    ids = np.array([1, 3, -1, 9, 0, 2, 0], np.int32)
    acc, _, written = R.int8_grouped(a, b, sa, sb, bias, offs, ids, raw=True)
    ref, tau, _ = R.int8_grouped(a, b, sa, sb, bias, offs, ids)
    show("grouped int8 ragged", k, with_bias)
    raw = torch.full((t, n), -7, dtype=torch.int32, device=DEV)
    _call(q, a, b, None, None, None, offs, ids, out=raw, out_dtype=torch.int32, max_tokens=r.integers(1, 3))
    got = raw.cpu().numpy()
    assert np.array_equal(got[written], acc[written].astype(np.int32))
    assert np.all(got[~written] == -7)
    out = torch.full((t, n), float("nan"), dtype=torch.float32, device=DEV)
    _call(q, a, b, sa, sb, bias, offs, ids, out=out, out_dtype=torch.float32, max_tokens=1)
    g = out.cpu().numpy()
    res = C.check_f32_tau(g[written], ref[written], tau[written])
    assert res, res
    assert np.all(np.isnan(g[~written]))


def test_grouped_int8_rejects_bad_arguments(q):
    a = torch.zeros((8, 64), dtype=torch.int8, device=DEV)
    b = torch.zeros((2, 16, 64), dtype=torch.int8, device=DEV)
    sa = torch.ones(8, dtype=torch.float32, device=DEV)
    sb = torch.ones(32, dtype=torch.float32, device=DEV)
    offs = torch.tensor([0, 8], dtype=torch.int32, device=DEV)
    ids = torch.tensor([1], dtype=torch.int32, device=DEV)
    out = torch.empty((8, 16), dtype=torch.bfloat16, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    f = q.lib.qlinear_int8_grouped_gemm
    show("grouped int8 bad args")
    assert f(p(a), p(b), p(sa), p(sb), None, p(offs), p(ids), p(out), 1, 1, 8, 2, 8, 16, 64, None) == 0
    assert f(p(a), p(b), None, p(sb), None, p(offs), p(ids), p(out), 1, 1, 8, 2, 8, 16, 64, None) == q.ERR_INVALID_ARG
    assert f(p(a), p(b), p(sa), p(sb), None, p(offs), p(ids), p(out), 5, 1, 8, 2, 8, 16, 64, None) == q.ERR_INVALID_ARG
    assert f(p(a), p(b), p(sa), p(sb), None, p(offs), p(ids), p(out), 1, 0, 8, 2, 8, 16, 64, None) == q.ERR_INVALID_ARG
    assert f(p(a), p(b), p(sa), p(sb), None, p(offs), p(ids), p(out), 1, 1, 8, 2, 8, 16, 200000,
             None) == q.ERR_INVALID_ARG
    odd = ctypes.c_void_p(sa.data_ptr() + 2)
    assert f(p(a), p(b), odd, p(sb), None, p(offs), p(ids), p(out), 1, 1, 8, 2, 8, 16, 64, None) == q.ERR_INVALID_ARG
    torch.cuda.synchronize()
