"""GPU parity of the LDS-tiled W8A16 GEMM and the grouped MoE W8A16 GEMM."""

import numpy as np
import pytest
import torch

import synth
from oracle import compare as C
from oracle import formats as F
from oracle import ref as R
from gpu_util import DEV, bf16_bits, show, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import weight_quantized_linear_amd as q
    return q


TILED_DYADIC = [(1, 1, 16), (17, 33, 48), (130, 257, 200), (256, 128, 4096), (300, 500, 2050),
                (129, 1, 64), (5, 1000, 4096), (128, 128, 13), (256, 128, 4032),
                # 256 x 128 tiles: 128-value strips (one; three, ragged M and N), 64-value strips
                # (K % 128 == 64); 256 x 256 tiles
                (2048, 4096, 128), (4100, 2100, 384), (2048, 4100, 192), (4096, 4096, 256),
                # split-K: nine 128-value strips over three slices; seventeen 64-value strips
                (128, 4096, 1152), (128, 4096, 1088)]


@pytest.mark.parametrize("m,n,k", TILED_DYADIC)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_tiled_dyadic_bit_exact(q, m, n, k, out_dtype):
    wc = synth.dyadic_fp8_weight((30, m, n, k), n, k)
    xc = synth.dyadic_activation((31, m, n, k), m, k)
    ref, _ = R.fp8_linear(wc, xc)
    show("tiled dyadic", m, n, k, out_dtype)
    out = q.fp8_gemm(to_dev_u8(wc), to_dev_bf16(xc), out_dtype=out_dtype, path="tiled")
    if out_dtype == torch.float32:
        assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))
    else:
        assert np.array_equal(bf16_bits(out), F.f64_to_bf16_bits(ref))


@pytest.mark.parametrize("m,n,k,out_dtype", [(2048, 1536, 2048, torch.float32), (64, 4096, 4096, torch.bfloat16),
                                             (333, 777, 1000, torch.float32)])
def test_tiled_realistic(q, m, n, k, out_dtype):
    w, s = synth.fp8_weight((32, m, n), n, k)
    x = synth.bf16_activation((33, m, n), m, k)
    ref, bound = R.fp8_linear(w, x, s)
    show("tiled realistic", m, n, k)
    out = q.fp8_gemm(to_dev_u8(w), to_dev_bf16(x), out_dtype=out_dtype, alpha=s)
    if out_dtype == torch.float32:
        res = C.check_f32(out.cpu().numpy(), ref, bound)
        assert res and res.max_rel < 1e-5, res
    else:
        res = C.check_bf16(bf16_bits(out), ref, C.fp_tolerance(bound))
        assert res and res.n_clause2 <= C.clause2_budget(ref), res


def test_tiled_and_skinny_agree_on_exact_inputs(q):
    wc = synth.dyadic_fp8_weight((34,), 999, 4096)
    xc = synth.dyadic_activation((35,), 16, 4096)
    w, x = to_dev_u8(wc), to_dev_bf16(xc)
    show("tiled vs skinny")
    a = q.fp8_gemm(w, x, out_dtype=torch.float32, path="tiled")
    b = q.fp8_gemm(w, x, out_dtype=torch.float32, path="skinny")
    assert torch.equal(a, b)


# ------------------------------------------------------------------ grouped

def _grouped(q, w, x, offs, ids, out=None, out_dtype=torch.bfloat16, max_tokens=None):
    # offsets travel as int32 bit patterns of the uint32 values (all < 2^31 here)
    return q.fp8_grouped_gemm(to_dev_u8(w), to_dev_bf16(x), torch.from_numpy(np.asarray(offs, np.int32)).to(DEV),
                              torch.from_numpy(np.asarray(ids, np.int32)).to(DEV), out=out, out_dtype=out_dtype,
                              max_tokens_per_group=max_tokens)


def test_grouped_moe_workload(q):
    c = synth.config4_case()
    t, n = c.x.shape[0], c.w.shape[1]
    show("grouped moe", c.name)
    out = torch.full((t, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    _grouped(q, c.w, c.x, c.a_offsets, c.expert_ids, out=out, max_tokens=c.max_tokens)
    torch.cuda.synchronize()
    ref, bound, written = R.fp8_grouped(c.w, c.x, c.a_offsets, c.expert_ids)
    got = bf16_bits(out)
    assert written.all()
    res = C.check_bf16(got, ref, C.fp_tolerance(bound))
    assert res and res.n_clause2 <= C.clause2_budget(ref), res
    inactive = np.zeros(t, bool)
    for z in np.flatnonzero(c.expert_ids == -1):
        inactive[c.a_offsets[z]:c.a_offsets[z + 1]] = True
    assert inactive.sum() == 40 and np.all(got[inactive] == 0)


def test_grouped_untouched_rows_and_guards(q):
    e, n, k, t = 4, 200, 96, 300
    w = synth.fp8_weight((41,), e * n, k)[0].reshape(e, n, k)
    x = synth.bf16_activation((42,), t, k)
    # rows 0..9 uncovered; group 1 empty; group 2 inactive (-1); group 3 id past E (zeros);
    # group 5 runs past T (clipped); group 6 has end < start (empty).  max_tokens (7) is
    # below every real group size: groups are still computed in full.
    offs = np.array([10, 60, 60, 90, 100, 260, 400, 150], np.int64)
    ids = np.array([1, 3, -1, 9, 0, 2, 0], np.int32)
    show("grouped guards")
    out = torch.full((t, n), float("nan"), dtype=torch.float32, device=DEV)
    _grouped(q, w, x, offs, ids, out=out, out_dtype=torch.float32, max_tokens=7)
    got = out.cpu().numpy()
    ref, bound, written = R.fp8_grouped(w, x, offs, ids)
    assert (~written).sum() == 10 and np.all(np.isnan(got[~written]))
    assert np.all(got[60:100] == 0)
    assert C.check_f32(got[written], ref[written], bound[written])


def test_grouped_single_group_equals_tiled(q):
    # Exactly representable sums: the two kernels add in different orders.
    w = synth.dyadic_fp8_weight((43,), 3 * 512, 1024).reshape(3, 512, 1024)
    x = synth.dyadic_activation((44,), 777, 1024)
    show("grouped single")
    g = _grouped(q, w, x, np.array([0, 777]), np.array([2]), out_dtype=torch.float32)
    d = q.fp8_gemm(to_dev_u8(np.ascontiguousarray(w[2])), to_dev_bf16(x), out_dtype=torch.float32, path="tiled")
    assert torch.equal(g, d)


# K % 64 != 0 (element-wise kernel), K % 128 == 64 (64-value strips), K % 128 == 0 (128-value strips)
@pytest.mark.parametrize("k", [2050, 192, 256])
def test_grouped_dyadic_bit_exact(q, k):
    e, n = 5, 130
    w = synth.dyadic_fp8_weight((45,), e * n, k).reshape(e, n, k)
    x = synth.dyadic_activation((46,), 401, k)
    offs = np.array([0, 1, 129, 129, 300, 401])
    ids = np.array([4, 0, 1, -1, 2], np.int32)
    ref, _, written = R.fp8_grouped(w, x, offs, ids)
    show("grouped dyadic", k)
    out = _grouped(q, w, x, offs, ids, out_dtype=torch.bfloat16, max_tokens=1)
    assert written.all()
    assert np.array_equal(bf16_bits(out), F.f64_to_bf16_bits(ref))


def test_grouped_rejects_bad_arguments(q):
    w = torch.zeros((2, 4, 16), dtype=torch.uint8, device=DEV)
    x = torch.zeros((3, 16), dtype=torch.bfloat16, device=DEV)
    offs = torch.zeros(3, dtype=torch.int32, device=DEV)
    ids = torch.zeros(3, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        q.fp8_grouped_gemm(w, x, offs, ids)  # a_offsets must have G + 1 entries
    st = q.lib.qlinear_fp8_grouped_gemm(w.data_ptr(), x.data_ptr(), offs.data_ptr(), ids.data_ptr(),
                                        x.data_ptr(), 0, 0, 1, 2, 3, 4, 16, None)
    assert st == q.ERR_INVALID_ARG  # zero groups
