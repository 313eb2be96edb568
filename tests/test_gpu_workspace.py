"""The caller-owned split-K workspace of the *_gemm_ws calls: the size query,
calls without a workspace (whole-K tiles), calls with a smaller one, two
calls running at once on two streams with their own workspaces, and a graph
captured before any eager call of its shapes; every result is checked
against the CPU oracle (bit for bit on exact inputs)."""

import ctypes

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


def test_workspace_size_query(q):
    """Split-K shapes ask for float32 partial planes [splits, M, N]; shapes
    with enough output tiles, the GEMV and the plain skinny kernel ask for none."""
    show("workspace size query")
    nv = q.gemm_workspace_bytes(q.WEIGHT_NVFP4, 128, 4096, 4096)
    assert nv > 0 and nv % (128 * 4096 * 4) == 0 and nv // (128 * 4096 * 4) >= 2
    sk = q.gemm_workspace_bytes(q.WEIGHT_FP8, 16, 4096, 14336)
    assert sk > 0 and sk % (16 * 4096 * 4) == 0
    assert q.gemm_workspace_bytes(q.WEIGHT_FP8, 64, 1000, 2048) > 0          # tiled split-K
    assert q.gemm_workspace_bytes(q.WEIGHT_FP8, 4096, 4096, 4096) == 0       # whole-K tiles
    assert q.gemm_workspace_bytes(q.WEIGHT_FP8, 1, 4096, 4096) == 0          # GEMV
    assert q.gemm_workspace_bytes(q.WEIGHT_FP8, 16, 4096, 4096) == 0         # skinny, K < 8192
    assert q.gemm_workspace_bytes(q.WEIGHT_NVFP4, 2048, 4096, 4096) == 0
    assert q.gemm_workspace_bytes(q.WEIGHT_BF16, 64, 1000, 2048) > 0
    assert q.gemm_workspace_bytes(q.WEIGHT_FP8, 12, 1000, 4096, path="splitk") > 0


CASES = [  # (kind, M, N, K): each takes split-K with a workspace
    ("fp8", 64, 1000, 2048),
    ("fp8", 16, 4096, 14336),
    ("nvfp4", 128, 4096, 4096),
    ("bf16", 40, 700, 2048),
]


def _dyadic(kind, key, m, n, k):
    x = synth.dyadic_activation(key + (1,), m, k)
    if kind == "fp8":
        w = synth.dyadic_fp8_weight(key, n, k)
        return (to_dev_u8(w),), x, R.fp8_linear(w, x)[0]
    if kind == "nvfp4":
        p, s = synth.dyadic_nvfp4_weight(key, n, k)
        return (to_dev_u8(p), to_dev_u8(s)), x, R.nvfp4_linear(p, s, x)[0]
    w = synth.dyadic_bf16_weight(key, n, k)
    return (to_dev_bf16(w),), x, R.bf16_linear(w, x)[0]


def _call(q, kind, wargs, x, out, workspace):
    fn = {"fp8": q.fp8_gemm, "nvfp4": q.nvfp4_gemm, "bf16": q.bf16_gemm}[kind]
    return fn(*wargs, x, out=out, out_dtype=out.dtype, workspace=workspace)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[1]}x{c[2]}x{c[3]}" for c in CASES])
def test_exact_with_full_partial_and_no_workspace(q, case):
    """Exact inputs: every split (full workspace, a workspace too small for
    the preferred split, none at all) gives the oracle's bits."""
    kind, m, n, k = case
    wargs, xb, ref = _dyadic(kind, (90, m, n, k), m, n, k)
    x = to_dev_bf16(xb)
    fmt = {"fp8": q.WEIGHT_FP8, "nvfp4": q.WEIGHT_NVFP4, "bf16": q.WEIGHT_BF16}[kind]
    need = q.gemm_workspace_bytes(fmt, m, n, k)
    assert need > 0
    small = torch.empty(max(16, (need // 2) // 16 * 16), dtype=torch.uint8, device=DEV)
    for ws in ("auto", small, None):
        show("workspace exact", kind, m, n, k, "none" if ws is None else ("auto" if isinstance(ws, str) else "small"))
        out = torch.full((m, n), float("nan"), dtype=torch.float32, device=DEV)
        _call(q, kind, wargs, x, out, ws)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))


def test_two_streams_with_own_workspaces(q):
    """Two split-K calls enqueued on two streams with no ordering between
    them, each with its own workspace: both results are the oracle's bits."""
    k1, k2 = CASES[0], CASES[2]
    w1, x1b, ref1 = _dyadic(k1[0], (91,), *k1[1:])
    w2, x2b, ref2 = _dyadic(k2[0], (92,), *k2[1:])
    x1, x2 = to_dev_bf16(x1b), to_dev_bf16(x2b)
    ws1 = torch.empty(q.gemm_workspace_bytes(q.WEIGHT_FP8, *k1[1:]), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty(q.gemm_workspace_bytes(q.WEIGHT_NVFP4, *k2[1:]), dtype=torch.uint8, device=DEV)
    o1 = torch.empty((k1[1], k1[2]), dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty((k2[1], k2[2]), dtype=torch.bfloat16, device=DEV)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    show("workspace two streams")
    for _ in range(4):
        with torch.cuda.stream(s1):
            _call(q, k1[0], w1, x1, o1, ws1)
        with torch.cuda.stream(s2):
            _call(q, k2[0], w2, x2, o2, ws2)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(o1), F.f64_to_bf16_bits(ref1))
    assert np.array_equal(bf16_bits(o2), F.f64_to_bf16_bits(ref2))


def test_graph_captured_first_matches_eager(q):
    """Shapes no earlier call used, captured into a graph before their first
    eager call: the replays equal the eager results bit for bit on realistic
    data (same kernels, same summation order), and both are within the
    tolerance of the oracle."""
    m, n, k = 48, 1536, 3072
    w, s = synth.fp8_weight((93,), n, k)
    xb = synth.bf16_activation((94,), m, k)
    packed, scales, g = synth.nvfp4_weight((95,), n, k)
    wd, x, pd, sd = to_dev_u8(w), to_dev_bf16(xb), to_dev_u8(packed), to_dev_u8(scales)
    outs = [torch.empty((m, n), dtype=torch.float32, device=DEV) for _ in range(2)]

    def work():
        q.fp8_gemm(wd, x, out=outs[0], out_dtype=torch.float32, alpha=float(s))
        q.nvfp4_gemm(pd, sd, x, out=outs[1], out_dtype=torch.float32, alpha=float(g))

    show("workspace graph first")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            work()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    replayed = [o.clone() for o in outs]
    for o in outs:
        o.zero_()
    work()
    torch.cuda.synchronize()
    for a, b in zip(replayed, outs):
        assert torch.equal(a, b)
    ref, bound = R.fp8_linear(w, xb, s)
    assert C.check_f32(outs[0].cpu().numpy(), ref, bound)
    ref, bound = R.nvfp4_linear(packed, scales, xb, float(g))
    assert C.check_f32(outs[1].cpu().numpy(), ref, bound)


def test_plain_calls_take_no_workspace(q):
    """The plain C calls (no workspace argument) run whole-K tiles: on exact
    inputs they give the oracle's bits at a split-K shape."""
    kind, m, n, k = CASES[2]
    (pd, sd), xb, ref = _dyadic(kind, (96,), m, n, k)
    x = to_dev_bf16(xb)
    out = torch.empty((m, n), dtype=torch.float32, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    show("workspace plain call")
    st = q.lib.qlinear_nvfp4_gemm(p(pd), p(sd), p(x), p(out), q.F32, m, n, k, 1.0,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == q.OK
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))
