"""Python binding of libqlinear, the MI355X (gfx950) weight-quantized linear
layer ``out = x @ dequant(W)^T``.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libqlinear.so``.  torch provides device memory and the current
stream.  There is no fallback: if the library is not built, importing this
package raises ImportError.

The C entry points (``include/qlinear.h``) are exposed unchanged as
``weight_quantized_linear_amd.lib.<name>``; the functions below take and
return torch tensors.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "lib",
    "LIB_PATH",
    "QLinearError",
    "EXPORTED",
    "fp8_gemv",
    "fp8_gemm",
    "bf16_gemm",
    "fp8_materialize",
    "fp8_grouped_gemm",
    "nvfp4_grouped_gemm",
    "int8_grouped_gemm",
    "fp8_quantize_act",
    "fp8_w8a8_gemm",
    "nvfp4_gemm",
    "nvfp4_dequant",
    "int8_quantize_act",
    "int8_gemm",
    "PATHS",
    "gemm_workspace_bytes",
    "WEIGHT_FP8",
    "WEIGHT_NVFP4",
    "WEIGHT_BF16",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlinear.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_DEVICE, ERR_LAUNCH, ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4, 5
F32, BF16, I32 = 0, 1, 2
PATHS = {"auto": 0, "gemv": 1, "skinny": 2, "tiled": 3, "splitk": 4}

_p, _i, _i64, _f = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float


class EpilogueDesc(ctypes.Structure):
    """``qlinear_epilogue``: the fused element-wise steps of the *_epilogue calls."""
    _fields_ = [("row_scale", _p), ("col_scale", _p), ("bias", _p), ("residual", _p),
                ("residual_ld", _i64), ("residual_dtype", _i), ("activation", _i)]


ACTIVATIONS = {"none": 0, "relu": 1, "silu": 2, "gelu_tanh": 3}
_EP = ctypes.POINTER(EpilogueDesc)

# name -> argument types (all return int status except where noted)
EXPORTED = {
    "qlinear_abi_version": [],
    "qlinear_status_string": [_i],
    "qlinear_fp8_gemv": [_p, _p, _p, _i, _i64, _i64, _f, _p],
    "qlinear_fp8_gemm": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _p],
    "qlinear_fp8_gemm_path": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _i, _p],
    "qlinear_bf16_gemm": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _p],
    "qlinear_bf16_gemm_path": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _i, _p],
    "qlinear_fp8_materialize": [_p, _p, _i, _i64, _i64, _p],
    "qlinear_fp8_grouped_gemm": [_p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _i64, _i64, _i64, _p],
    "qlinear_nvfp4_gemm": [_p, _p, _p, _p, _i, _i64, _i64, _i64, _f, _p],
    "qlinear_nvfp4_grouped_gemm": [_p, _p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _i64, _i64, _i64, _p],
    "qlinear_fp8_quantize_act": [_p, _p, _f, _i64, _i64, _p],
    "qlinear_fp8_w8a8_gemm": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _p],
    "qlinear_nvfp4_gemm_path": [_p, _p, _p, _p, _i, _i64, _i64, _i64, _f, _i, _p],
    "qlinear_nvfp4_dequant": [_p, _p, _p, _i, _i64, _i64, _p],
    "qlinear_int8_quantize_act": [_p, _p, _p, _i64, _i64, _p],
    "qlinear_int8_gemm": [_p, _p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _p],
    "qlinear_fp8_gemm_epilogue": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _EP, _p],
    "qlinear_fp8_gemm_epilogue_path": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _EP, _i, _p],
    "qlinear_nvfp4_gemm_epilogue": [_p, _p, _p, _p, _i, _i64, _i64, _i64, _f, _EP, _p],
    "qlinear_bf16_gemm_epilogue": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _EP, _p],
    "qlinear_fp8_grouped_gemm_scaled": [_p, _p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _i64, _i64, _i64, _p],
    "qlinear_nvfp4_grouped_gemm_scaled": [_p, _p, _p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _i64, _i64, _i64, _p],
    "qlinear_int8_grouped_gemm": [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _i64, _i64, _i64, _p],
    "qlinear_gemm_workspace_size": [_i, _i, _i64, _i64, _i64, ctypes.POINTER(_i64)],
    "qlinear_fp8_gemm_ws": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _EP, _i, _p, _i64, _p],
    "qlinear_nvfp4_gemm_ws": [_p, _p, _p, _p, _i, _i64, _i64, _i64, _f, _EP, _i, _p, _i64, _p],
    "qlinear_bf16_gemm_ws": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _EP, _i, _p, _i64, _p],
    "qlinear_fp8_gemm_noalloc": [_p, _p, _p, _i, _i64, _i64, _i64, _f, _EP, _i, _p],
}

WEIGHT_FP8, WEIGHT_NVFP4, WEIGHT_BF16 = 0, 1, 2


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python weight_quantized_linear_amd/build.py`")
    handle = ctypes.CDLL(LIB_PATH)
    for name, argtypes in EXPORTED.items():
        fn = getattr(handle, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_char_p if name == "qlinear_status_string" else _i
    return handle


lib = _load()


class QLinearError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {lib.qlinear_status_string(status).decode()} (status {status})")


def _check(status: int, call: str):
    if status != OK:
        raise QLinearError(status, call)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _as_u8(w: torch.Tensor, what: str) -> torch.Tensor:
    if w.dtype in (torch.uint8, torch.int8):
        return w
    if w.dtype == torch.float8_e4m3fn:
        return w.view(torch.uint8)
    raise TypeError(f"{what}: expected float8_e4m3fn/uint8 storage, got {w.dtype}")


def _as_bf16(x: torch.Tensor, what: str) -> torch.Tensor:
    if x.dtype == torch.bfloat16:
        return x
    if x.dtype in (torch.int16, torch.uint16):
        return x.view(torch.bfloat16)
    raise TypeError(f"{what}: expected bfloat16 storage, got {x.dtype}")


def _require(t: torch.Tensor, what: str):
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


_OUT_CODES = {torch.float32: F32, torch.bfloat16: BF16}


def _out(out, shape, dtype, device):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _require(out, "out")
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype:
        raise ValueError(f"out must be {tuple(shape)} {dtype}, got {tuple(out.shape)} {out.dtype}")
    return out


def _epilogue(m: int, n: int, row_scale, col_scale, bias, residual, activation: str):
    """The ``qlinear_epilogue`` of the given tensors (None when nothing is fused)."""
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}")
    if row_scale is None and col_scale is None and bias is None and residual is None and activation == "none":
        return None
    d = EpilogueDesc(None, None, None, None, 0, F32, ACTIVATIONS[activation])
    for t, name, size, dt in ((row_scale, "row_scale", m, torch.float32), (col_scale, "col_scale", n, torch.float32),
                              (bias, "bias", n, torch.bfloat16)):
        if t is None:
            continue
        _require(t, name)
        if t.dtype != dt or t.numel() != size:
            raise ValueError(f"{name} must be {dt} with {size} elements")
        setattr(d, name, t.data_ptr())
    if residual is not None:
        if not residual.is_cuda or residual.dim() != 2 or residual.shape[0] != m or residual.shape[1] < n \
                or residual.stride(1) != 1 or residual.dtype not in _OUT_CODES:
            raise ValueError("residual must be a float32/bfloat16 device tensor [M, >= N] with unit column stride")
        d.residual = residual.data_ptr()
        d.residual_ld = residual.stride(0) if m > 1 else residual.shape[1]
        d.residual_dtype = _OUT_CODES[residual.dtype]
    return d


def _epi_ref(d):
    return ctypes.byref(d) if d is not None else None


def gemm_workspace_bytes(weight_format: int, m: int, n: int, k: int, path: str = "auto") -> int:
    """Bytes of split-K workspace the ``*_gemm_ws`` call of ``weight_format``
    (WEIGHT_FP8 / WEIGHT_NVFP4 / WEIGHT_BF16) takes for (m, n, k) on the
    current device (``qlinear_gemm_workspace_size``); 0 = none."""
    b = _i64(0)
    _check(lib.qlinear_gemm_workspace_size(weight_format, PATHS[path], m, n, k, ctypes.byref(b)),
           "qlinear_gemm_workspace_size")
    return int(b.value)


def _workspace(workspace, weight_format: int, m: int, n: int, k: int, path: str, device):
    """(pointer, bytes, tensor) of the split-K workspace: "auto" allocates what
    the call takes (a torch tensor, so torch's caching allocator serves it),
    None passes none (whole-K tiles), a tensor is used as given."""
    if workspace is None:
        return None, 0, None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a device tensor")
        nbytes = gemm_workspace_bytes(weight_format, m, n, k, path)
        if nbytes == 0:
            return None, 0, None
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _require(workspace, "workspace")
    return _ptr(workspace), workspace.numel() * workspace.element_size(), workspace


def fp8_gemm(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
             out_dtype: torch.dtype = torch.bfloat16, alpha: float = 1.0, path: str = "auto",
             row_scale: torch.Tensor | None = None, col_scale: torch.Tensor | None = None,
             bias: torch.Tensor | None = None, residual: torch.Tensor | None = None,
             activation: str = "none", workspace="auto") -> torch.Tensor:
    """out[M, N] = alpha * x[M, K] @ dec_e4m3(w[N, K])^T (``qlinear_fp8_gemm_ws``), with
    the fused epilogue of any of row_scale / col_scale / bias / residual / activation,
    the kernel family ``path`` and the split-K ``workspace`` ("auto": allocated to the
    size ``qlinear_gemm_workspace_size`` gives; None: none)."""
    w = _as_u8(w, "w")
    x = _as_bf16(x, "x")
    _require(w, "w")
    _require(x, "x")
    if w.dim() != 2 or x.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"shapes: w {tuple(w.shape)} must be [N, K], x {tuple(x.shape)} must be [M, K]")
    m, k = x.shape
    n = w.shape[0]
    out = _out(out, (m, n), out_dtype, x.device)
    d = _epilogue(m, n, row_scale, col_scale, bias, residual, activation)
    wsp, wsb, _keep = _workspace(workspace, WEIGHT_FP8, m, n, k, path, x.device)
    st = lib.qlinear_fp8_gemm_ws(_ptr(w), _ptr(x), _ptr(out), _OUT_CODES[out_dtype], m, n, k, float(alpha),
                                 _epi_ref(d), PATHS[path], wsp, wsb, _stream(x))
    _check(st, "qlinear_fp8_gemm_ws")
    return out


def bf16_gemm(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
              out_dtype: torch.dtype = torch.bfloat16, alpha: float = 1.0, path: str = "auto",
              row_scale: torch.Tensor | None = None, col_scale: torch.Tensor | None = None,
              bias: torch.Tensor | None = None, residual: torch.Tensor | None = None,
              activation: str = "none", workspace="auto") -> torch.Tensor:
    """Dense bf16 control: out[M, N] = alpha * x[M, K] @ w[N, K]^T (``qlinear_bf16_gemm_ws``);
    epilogue, ``path`` and ``workspace`` as ``fp8_gemm``."""
    w = _as_bf16(w, "w")
    x = _as_bf16(x, "x")
    _require(w, "w")
    _require(x, "x")
    if w.dim() != 2 or x.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"shapes: w {tuple(w.shape)} must be [N, K], x {tuple(x.shape)} must be [M, K]")
    m, k = x.shape
    n = w.shape[0]
    out = _out(out, (m, n), out_dtype, x.device)
    d = _epilogue(m, n, row_scale, col_scale, bias, residual, activation)
    wsp, wsb, _keep = _workspace(workspace, WEIGHT_BF16, m, n, k, path, x.device)
    st = lib.qlinear_bf16_gemm_ws(_ptr(w), _ptr(x), _ptr(out), _OUT_CODES[out_dtype], m, n, k, float(alpha),
                                  _epi_ref(d), PATHS[path], wsp, wsb, _stream(x))
    _check(st, "qlinear_bf16_gemm_ws")
    return out


def fp8_gemv(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
             out_dtype: torch.dtype = torch.float32, alpha: float = 1.0) -> torch.Tensor:
    """out[N] = alpha * dec_e4m3(w[N, K]) @ x[K] (``qlinear_fp8_gemv``)."""
    w = _as_u8(w, "w")
    x = _as_bf16(x, "x")
    _require(w, "w")
    _require(x, "x")
    if w.dim() != 2 or x.numel() != w.shape[1]:
        raise ValueError("w must be [N, K] and x must hold K elements")
    n, k = w.shape
    out = _out(out, (n,), out_dtype, x.device)
    st = lib.qlinear_fp8_gemv(_ptr(w), _ptr(x), _ptr(out), _OUT_CODES[out_dtype], n, k, float(alpha), _stream(x))
    _check(st, "qlinear_fp8_gemv")
    return out


def fp8_materialize(w: torch.Tensor, out_dtype: torch.dtype = torch.float32,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense [N, K] copy of the decoded FP8 weight (``qlinear_fp8_materialize``)."""
    w = _as_u8(w, "w")
    _require(w, "w")
    w2 = w.reshape(1, -1) if w.dim() == 1 else w
    n, k = w2.shape
    out = _out(out, tuple(w.shape), out_dtype, w.device)
    st = lib.qlinear_fp8_materialize(_ptr(w2), _ptr(out), _OUT_CODES[out_dtype], n, k, _stream(w))
    _check(st, "qlinear_fp8_materialize")
    return out


def _expert_scale(expert_scale, e: int):
    if expert_scale is None:
        return None
    _require(expert_scale, "expert_scale")
    if expert_scale.dtype != torch.float32 or expert_scale.numel() != e:
        raise ValueError(f"expert_scale must be float32 with {e} elements")
    return _ptr(expert_scale)


def fp8_grouped_gemm(w: torch.Tensor, x: torch.Tensor, a_offsets: torch.Tensor, expert_ids: torch.Tensor,
                     out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
                     max_tokens_per_group: int | None = None,
                     expert_scale: torch.Tensor | None = None) -> torch.Tensor:
    """Grouped MoE W8A16 (``qlinear_fp8_grouped_gemm_scaled``): rows a_offsets[z] ..
    a_offsets[z+1]-1 of x times dec(w[expert_ids[z]])^T, times expert_scale[expert_ids[z]]
    when given (raw otherwise).  Rows outside every group keep whatever ``out`` held
    (a new ``out`` starts uninitialised)."""
    w = _as_u8(w, "w")
    x = _as_bf16(x, "x")
    for t, name in ((w, "w"), (x, "x"), (a_offsets, "a_offsets"), (expert_ids, "expert_ids")):
        _require(t, name)
    if a_offsets.dtype not in (torch.int32, torch.uint32) or expert_ids.dtype != torch.int32:
        raise TypeError("a_offsets must be uint32/int32 and expert_ids int32")
    if w.dim() != 3 or x.dim() != 2 or x.shape[1] != w.shape[2]:
        raise ValueError("w must be [E, N, K] and x [T, K]")
    g = expert_ids.numel()
    if a_offsets.numel() != g + 1:
        raise ValueError("a_offsets needs num_groups + 1 entries")
    e, n, k = w.shape
    t = x.shape[0]
    if max_tokens_per_group is None:
        max_tokens_per_group = t
    out = _out(out, (t, n), out_dtype, x.device)
    st = lib.qlinear_fp8_grouped_gemm_scaled(_ptr(w), _ptr(x), _ptr(a_offsets), _ptr(expert_ids),
                                             _expert_scale(expert_scale, e), _ptr(out), _OUT_CODES[out_dtype], g,
                                             int(max_tokens_per_group), e, t, n, k, _stream(x))
    _check(st, "qlinear_fp8_grouped_gemm_scaled")
    return out


def fp8_quantize_act(x: torch.Tensor, input_scale: float, q: torch.Tensor | None = None) -> torch.Tensor:
    """Static per-tensor FP8 activation quantisation (``qlinear_fp8_quantize_act``):
    q = E4M3(clamp(x / input_scale, -448, 448)) as uint8 codes [M, K]."""
    x = _as_bf16(x, "x")
    _require(x, "x")
    m, k = x.shape
    if q is None:
        q = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    elif q.dtype != torch.uint8 or tuple(q.shape) != (m, k) or not q.is_contiguous():
        raise ValueError("q must be a contiguous uint8 [M, K] tensor")
    st = lib.qlinear_fp8_quantize_act(_ptr(x), _ptr(q), float(input_scale), m, k, _stream(x))
    _check(st, "qlinear_fp8_quantize_act")
    return q


def fp8_w8a8_gemm(xq: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None,
                  out_dtype: torch.dtype = torch.bfloat16, alpha: float = 1.0) -> torch.Tensor:
    """FP8 W8A8 (``qlinear_fp8_w8a8_gemm``): out = alpha * dec(xq) @ dec(w)^T,
    xq and w float8_e4m3fn codes (uint8 or float8 tensors)."""
    xq = _as_u8(xq, "xq")
    w = _as_u8(w, "w")
    for t, name in ((xq, "xq"), (w, "w")):
        _require(t, name)
    m, k = xq.shape
    n = w.shape[0]
    if w.shape[1] != k:
        raise ValueError("xq must be [M, K] and w [N, K]")
    out = _out(out, (m, n), out_dtype, xq.device)
    st = lib.qlinear_fp8_w8a8_gemm(_ptr(xq), _ptr(w), _ptr(out), _OUT_CODES[out_dtype], m, n, k, float(alpha),
                                   _stream(xq))
    _check(st, "qlinear_fp8_w8a8_gemm")
    return out


def nvfp4_grouped_gemm(w_packed: torch.Tensor, w_scale: torch.Tensor, x: torch.Tensor, a_offsets: torch.Tensor,
                       expert_ids: torch.Tensor, out: torch.Tensor | None = None,
                       out_dtype: torch.dtype = torch.bfloat16, max_tokens_per_group: int | None = None,
                       expert_scale: torch.Tensor | None = None) -> torch.Tensor:
    """Grouped MoE W4A16 NVFP4 (``qlinear_nvfp4_grouped_gemm_scaled``): rows a_offsets[z] ..
    a_offsets[z+1]-1 of x times D_e^T, e = expert_ids[z], D_e the expert's NVFP4
    weight (w_packed [E, N, K/2], w_scale [E, N, K/16]), times expert_scale[e] when
    given (raw otherwise).  Rows outside every group keep whatever ``out`` held (a
    new ``out`` starts uninitialised)."""
    p = _as_u8(w_packed, "w_packed")
    sc = _as_u8(w_scale, "w_scale")
    x = _as_bf16(x, "x")
    for t, name in ((p, "w_packed"), (sc, "w_scale"), (x, "x"), (a_offsets, "a_offsets"), (expert_ids, "expert_ids")):
        _require(t, name)
    if a_offsets.dtype not in (torch.int32, torch.uint32) or expert_ids.dtype != torch.int32:
        raise TypeError("a_offsets must be uint32/int32 and expert_ids int32")
    if p.dim() != 3 or x.dim() != 2:
        raise ValueError("w_packed must be [E, N, K/2] and x [T, K]")
    e, n, _ = p.shape
    t, k = x.shape
    if tuple(p.shape) != (e, n, k // 2) or tuple(sc.shape) != (e, n, k // 16):
        raise ValueError("w_packed must be [E, N, K/2] and w_scale [E, N, K/16]")
    g = expert_ids.numel()
    if a_offsets.numel() != g + 1:
        raise ValueError("a_offsets needs num_groups + 1 entries")
    if max_tokens_per_group is None:
        max_tokens_per_group = t
    out = _out(out, (t, n), out_dtype, x.device)
    st = lib.qlinear_nvfp4_grouped_gemm_scaled(_ptr(p), _ptr(sc), _ptr(x), _ptr(a_offsets), _ptr(expert_ids),
                                               _expert_scale(expert_scale, e), _ptr(out), _OUT_CODES[out_dtype], g,
                                               int(max_tokens_per_group), e, t, n, k, _stream(x))
    _check(st, "qlinear_nvfp4_grouped_gemm_scaled")
    return out


def nvfp4_gemm(w_packed: torch.Tensor, w_scale: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
               out_dtype: torch.dtype = torch.bfloat16, alpha: float = 1.0, path: str = "auto",
               row_scale: torch.Tensor | None = None, col_scale: torch.Tensor | None = None,
               bias: torch.Tensor | None = None, residual: torch.Tensor | None = None,
               activation: str = "none", workspace="auto") -> torch.Tensor:
    """out[M, N] = alpha * x[M, K] @ D^T, D the NVFP4 weight (``qlinear_nvfp4_gemm_ws``);
    epilogue, ``path`` and ``workspace`` as ``fp8_gemm``."""
    p = _as_u8(w_packed, "w_packed")
    sc = _as_u8(w_scale, "w_scale")
    x = _as_bf16(x, "x")
    for t, name in ((p, "w_packed"), (sc, "w_scale"), (x, "x")):
        _require(t, name)
    m, k = x.shape
    n = p.shape[0]
    if tuple(p.shape) != (n, k // 2) or tuple(sc.shape) != (n, k // 16):
        raise ValueError("w_packed must be [N, K/2] and w_scale [N, K/16]")
    out = _out(out, (m, n), out_dtype, x.device)
    d = _epilogue(m, n, row_scale, col_scale, bias, residual, activation)
    wsp, wsb, _keep = _workspace(workspace, WEIGHT_NVFP4, m, n, k, path, x.device)
    st = lib.qlinear_nvfp4_gemm_ws(_ptr(p), _ptr(sc), _ptr(x), _ptr(out), _OUT_CODES[out_dtype], m, n, k,
                                   float(alpha), _epi_ref(d), PATHS[path], wsp, wsb, _stream(x))
    _check(st, "qlinear_nvfp4_gemm_ws")
    return out


def nvfp4_dequant(w_packed: torch.Tensor, w_scale: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense [N, K] dequantised NVFP4 weight (``qlinear_nvfp4_dequant``)."""
    p = _as_u8(w_packed, "w_packed")
    sc = _as_u8(w_scale, "w_scale")
    _require(p, "w_packed")
    _require(sc, "w_scale")
    n, half = p.shape
    k = 2 * half
    if tuple(sc.shape) != (n, k // 16):
        raise ValueError("w_scale must be [N, K/16]")
    out = _out(out, (n, k), out_dtype, p.device)
    st = lib.qlinear_nvfp4_dequant(_ptr(p), _ptr(sc), _ptr(out), _OUT_CODES[out_dtype], n, k, _stream(p))
    _check(st, "qlinear_nvfp4_dequant")
    return out


def int8_quantize_act(x: torch.Tensor, q: torch.Tensor | None = None, a_scale: torch.Tensor | None = None):
    """Per-row absmax int8 quantisation (``qlinear_int8_quantize_act``) -> (q int8 [M, K], a_scale f32 [M])."""
    x = _as_bf16(x, "x")
    _require(x, "x")
    m, k = x.shape
    q = _out(q, (m, k), torch.int8, x.device)
    a_scale = _out(a_scale, (m,), torch.float32, x.device)
    st = lib.qlinear_int8_quantize_act(_ptr(x), _ptr(q), _ptr(a_scale), m, k, _stream(x))
    _check(st, "qlinear_int8_quantize_act")
    return q, a_scale


_INT8_OUT = {torch.float32: F32, torch.bfloat16: BF16, torch.int32: I32}


def int8_gemm(a: torch.Tensor, b: torch.Tensor, a_scale: torch.Tensor | None, b_scale: torch.Tensor | None,
              bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
              out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """W8A8: out = (a @ b^T) * a_scale[:, None] * b_scale[None, :] + bias (``qlinear_int8_gemm``);
    out_dtype=torch.int32 returns the raw accumulators."""
    for t, name in ((a, "a"), (b, "b")):
        _require(t, name)
        if t.dtype != torch.int8:
            raise TypeError(f"{name} must be int8")
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k:
        raise ValueError("a must be [M, K] and b [N, K]")
    args = []
    for t, name, shape in ((a_scale, "a_scale", (m,)), (b_scale, "b_scale", (n,))):
        if t is None:
            args.append(None)
            continue
        _require(t, name)
        if t.dtype != torch.float32 or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be float32 {shape}")
        args.append(_ptr(t))
    bias_p = None
    if bias is not None:
        bias = _as_bf16(bias, "bias")
        _require(bias, "bias")
        if tuple(bias.shape) != (n,):
            raise ValueError("bias must be [N]")
        bias_p = _ptr(bias)
    out = _out(out, (m, n), out_dtype, a.device)
    st = lib.qlinear_int8_gemm(_ptr(a), _ptr(b), args[0], args[1], bias_p, _ptr(out), _INT8_OUT[out_dtype],
                               m, n, k, _stream(a))
    _check(st, "qlinear_int8_gemm")
    return out


def int8_grouped_gemm(a: torch.Tensor, b: torch.Tensor, a_scale: torch.Tensor | None, b_scale: torch.Tensor | None,
                      a_offsets: torch.Tensor, expert_ids: torch.Tensor, bias: torch.Tensor | None = None,
                      out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
                      max_tokens_per_group: int | None = None) -> torch.Tensor:
    """Grouped MoE W8A8 (``qlinear_int8_grouped_gemm``): rows a_offsets[z] ..
    a_offsets[z+1]-1 of the int8 activation a [T, K] times b[expert_ids[z]] [N, K]^T,
    dequantised by a_scale[r] * b_scale[e, n] + bias[e, n] (out_dtype bf16 / f32) or
    raw int32 accumulators (out_dtype int32).  Rows outside every group keep whatever
    ``out`` held (a new ``out`` starts uninitialised)."""
    codes = {torch.float32: F32, torch.bfloat16: BF16, torch.int32: I32}
    if out_dtype not in codes:
        raise ValueError("out_dtype must be bfloat16, float32 or int32")
    for t, name in ((a, "a"), (b, "b"), (a_offsets, "a_offsets"), (expert_ids, "expert_ids")):
        _require(t, name)
    if a.dtype != torch.int8 or b.dtype != torch.int8:
        raise TypeError("a and b must be int8")
    if a_offsets.dtype not in (torch.int32, torch.uint32) or expert_ids.dtype != torch.int32:
        raise TypeError("a_offsets must be uint32/int32 and expert_ids int32")
    if b.dim() != 3 or a.dim() != 2 or a.shape[1] != b.shape[2]:
        raise ValueError("b must be [E, N, K] and a [T, K]")
    e, n, k = b.shape
    t = a.shape[0]
    g = expert_ids.numel()
    if a_offsets.numel() != g + 1:
        raise ValueError("a_offsets needs num_groups + 1 entries")
    if out_dtype != torch.int32:
        if a_scale is None or b_scale is None:
            raise ValueError("a_scale and b_scale are needed for a dequantised output")
        for s_, name, size in ((a_scale, "a_scale", t), (b_scale, "b_scale", e * n)):
            _require(s_, name)
            if s_.dtype != torch.float32 or s_.numel() != size:
                raise ValueError(f"{name} must be float32 with {size} elements")
        if bias is not None:
            _require(bias, "bias")
            if bias.dtype != torch.bfloat16 or bias.numel() != e * n:
                raise ValueError(f"bias must be bfloat16 with {e * n} elements")
    if max_tokens_per_group is None:
        max_tokens_per_group = t
    out = _out(out, (t, n), out_dtype, a.device)
    opt = lambda x: None if x is None else _ptr(x)  # noqa: E731
    st = lib.qlinear_int8_grouped_gemm(_ptr(a), _ptr(b), opt(a_scale), opt(b_scale), opt(bias), _ptr(a_offsets),
                                       _ptr(expert_ids), _ptr(out), codes[out_dtype], g, int(max_tokens_per_group),
                                       e, t, n, k, _stream(a))
    _check(st, "qlinear_int8_grouped_gemm")
    return out

