"""GPU parity of the grouped MoE W4A16 NVFP4 call (qlinear_nvfp4_grouped_gemm)
against the CPU oracle, through the C ABI."""

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


def _grouped(q, packed, scales, x, offs, ids, out=None, out_dtype=torch.bfloat16, max_tokens=None):
    # offsets travel as int32 bit patterns of the uint32 values (all < 2^31 here)
    return q.nvfp4_grouped_gemm(to_dev_u8(packed), to_dev_u8(scales), to_dev_bf16(x),
                                torch.from_numpy(np.asarray(offs, np.int32)).to(DEV),
                                torch.from_numpy(np.asarray(ids, np.int32)).to(DEV), out=out, out_dtype=out_dtype,
                                max_tokens_per_group=max_tokens)


def _dyadic_stack(key, e, n, k):
    p, s = synth.dyadic_nvfp4_weight(key, e * n, k)
    return p.reshape(e, n, k // 2), s.reshape(e, n, k // 16)


def test_grouped_nvfp4_workload(q):
    c = synth.grouped_nvfp4_case()
    t, n = c.x.shape[0], c.packed.shape[1]
    show("grouped nvfp4 workload", c.name)
    out = torch.full((t, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    _grouped(q, c.packed, c.scales, c.x, c.a_offsets, c.expert_ids, out=out, max_tokens=c.max_tokens)
    torch.cuda.synchronize()
    ref, bound, written = R.nvfp4_grouped(c.packed, c.scales, c.x, c.a_offsets, c.expert_ids)
    got = bf16_bits(out)
    assert written.all()
    res = C.check_bf16(got, ref, C.fp_tolerance(bound))
    assert res and res.n_clause2 <= C.clause2_budget(ref), res
    inactive = np.zeros(t, bool)
    for z in np.flatnonzero(c.expert_ids == -1):
        inactive[c.a_offsets[z]:c.a_offsets[z + 1]] = True
    assert inactive.sum() == 40 and np.all(got[inactive] == 0)


# LDS path (128-value strips, then 64-value strips); element-wise path (K % 64 != 0, then K % 32 != 0)
@pytest.mark.parametrize("k", [2048, 192, 2080, 1040])
def test_grouped_nvfp4_dyadic_bit_exact(q, k):
    e, n = 5, 130
    p, s = _dyadic_stack((70, k), e, n, k)
    x = synth.dyadic_activation((71, k), 401, k)
    offs = np.array([0, 1, 129, 129, 300, 401])
    ids = np.array([4, 0, 1, -1, 2], np.int32)
    ref, _, written = R.nvfp4_grouped(p, s, x, offs, ids)
    show("grouped nvfp4 dyadic", k)
    out = _grouped(q, p, s, x, offs, ids, out_dtype=torch.bfloat16, max_tokens=1)
    assert written.all()
    assert np.array_equal(bf16_bits(out), F.f64_to_bf16_bits(ref))
    out32 = _grouped(q, p, s, x, offs, ids, out_dtype=torch.float32, max_tokens=1)
    assert np.array_equal(out32.cpu().numpy(), ref.astype(np.float32))


def test_grouped_nvfp4_untouched_rows_and_guards(q):
    e, n, k, t = 4, 200, 128, 300
    p, s, _ = synth.nvfp4_weight((72,), e * n, k)
    p, s = p.reshape(e, n, k // 2), s.reshape(e, n, k // 16)
    x = synth.bf16_activation((73,), t, k)
    # rows 0..9 uncovered; group 1 empty; group 2 inactive; group 3 id past E;
    # group 5 runs past T (clipped); group 6 has end < start (empty).
    offs = np.array([10, 60, 60, 90, 100, 260, 400, 150], np.int64)
    ids = np.array([1, 3, -1, 9, 0, 2, 0], np.int32)
    show("grouped nvfp4 guards")
    out = torch.full((t, n), float("nan"), dtype=torch.float32, device=DEV)
    _grouped(q, p, s, x, offs, ids, out=out, out_dtype=torch.float32, max_tokens=7)
    got = out.cpu().numpy()
    ref, bound, written = R.nvfp4_grouped(p, s, x, offs, ids)
    assert (~written).sum() == 10 and np.all(np.isnan(got[~written]))
    assert np.all(got[60:100] == 0)
    assert C.check_f32(got[written], ref[written], bound[written])


def test_grouped_nvfp4_single_group_equals_tiled(q):
    # Exactly representable sums: the two kernels add in different orders.
    p, s = _dyadic_stack((74,), 3, 512, 1024)
    x = synth.dyadic_activation((75,), 777, 1024)
    show("grouped nvfp4 single")
    g = _grouped(q, p, s, x, np.array([0, 777]), np.array([2]), out_dtype=torch.float32)
    d = q.nvfp4_gemm(to_dev_u8(np.ascontiguousarray(p[2])), to_dev_u8(np.ascontiguousarray(s[2])), to_dev_bf16(x),
                     out_dtype=torch.float32, path="tiled")
    assert torch.equal(g, d)


def test_grouped_nvfp4_rejects_bad_arguments(q):
    p = torch.zeros((2, 4, 8), dtype=torch.uint8, device=DEV)
    s = torch.zeros((2, 4, 1), dtype=torch.uint8, device=DEV)
    x = torch.zeros((3, 16), dtype=torch.bfloat16, device=DEV)
    offs = torch.zeros(3, dtype=torch.int32, device=DEV)
    ids = torch.zeros(2, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        q.nvfp4_grouped_gemm(p, s, x, offs[:2], ids)  # a_offsets must have G + 1 entries
    st = q.lib.qlinear_nvfp4_grouped_gemm(p.data_ptr(), s.data_ptr(), x.data_ptr(), offs.data_ptr(), ids.data_ptr(),
                                          x.data_ptr(), 0, 2, 3, 2, 3, 4, 24, None)
    assert st == q.ERR_INVALID_ARG  # K % 16 != 0
