"""qlinear_fp8_gemm_noalloc (split-K partial sums in the library's fixed
device buffer, no allocation) against qlinear_fp8_gemm_ws with a
caller-allocated workspace, through the C ABI: bit-identical outputs on two
calls in a row, the second smaller, both within the oracle's tolerance; a
shape that needs more than the buffer is refused and writes nothing."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import compare as C
from oracle import ref as R
from gpu_util import DEV, show, to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 8 << 20


@pytest.fixture(scope="module")
def q():
    import weight_quantized_linear_amd as q
    return q


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _noalloc(q, w, x, out, alpha, path=0):
    m, k = x.shape
    n = w.shape[0]
    code = q.F32 if out.dtype == torch.float32 else q.BF16
    return q.lib.qlinear_fp8_gemm_noalloc(_p(w), _p(x), _p(out), code, m, n, k, float(alpha), None, path,
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


# (M, N, K, out dtype): split-K skinny, then a smaller split-K tiled shape,
# then the smallest split-K skinny shape and a call with no split-K at all
SEQUENCE = [(16, 4096, 14336, torch.bfloat16), (40, 1000, 2048, torch.float32),
            (12, 300, 8192, torch.float32), (1, 2048, 2048, torch.float32)]


def test_noalloc_matches_workspace_call(q):
    sizes = []
    for i, (m, n, k, dt) in enumerate(SEQUENCE):
        w, s = synth.fp8_weight((97, i), n, k)
        xb = synth.bf16_activation((98, i), m, k)
        wd, x = to_dev_u8(w), to_dev_bf16(xb)
        need = q.gemm_workspace_bytes(q.WEIGHT_FP8, m, n, k)
        assert need <= SCRATCH_BYTES
        sizes.append(need)
        show("noalloc", i, m, n, k, dt, need)
        ref_out = q.fp8_gemm(wd, x, out_dtype=dt, alpha=float(s))          # caller-allocated workspace
        out = torch.full((m, n), float("nan"), dtype=dt, device=DEV)
        assert _noalloc(q, wd, x, out, s) == q.OK
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), (m, n, k)
        ref, bound = R.fp8_linear(w, xb, s)
        if dt == torch.float32:
            assert C.check_f32(out.cpu().numpy(), ref, bound)
        else:
            bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
            res = C.check_bf16(bits, ref, C.fp_tolerance(bound))
            assert res and res.n_clause2 <= C.clause2_budget(ref), res
    assert sizes[0] > sizes[1] > 0 and sizes[2] > 0 and sizes[3] == 0


def test_noalloc_refuses_shapes_beyond_its_buffer(q):
    m, n, k = 128, 1024, 8192
    need = q.gemm_workspace_bytes(q.WEIGHT_FP8, m, n, k)
    if need <= SCRATCH_BYTES:
        pytest.skip(f"this device's split for {m}x{n}x{k} fits the buffer ({need} bytes)")
    w = torch.zeros((n, k), dtype=torch.uint8, device=DEV)
    x = torch.zeros((m, k), dtype=torch.bfloat16, device=DEV)
    out = torch.full((m, n), 3.0, dtype=torch.float32, device=DEV)
    show("noalloc refuses", m, n, k, need)
    assert _noalloc(q, w, x, out, 1.0) == q.ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
