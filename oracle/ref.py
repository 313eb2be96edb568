"""Reference results of the weight-quantized linear layer, by definition.

Test infrastructure (see the package docstring): the HIP library never imports
this module.

Every float result is ``sum_k x[m,k] * w[n,k]`` over exactly decoded operands,
evaluated as a float64 matrix product (numpy/BLAS is the only library step).
Alongside each result the functions return the magnitude sum
``B[m,n] = |alpha| * sum_k |x[m,k] * w[n,k]|`` that the acceptance rule of
``oracle.compare`` scales its tolerance by.  Integer results are exact.

Inputs are the raw stored codes, exactly as the kernels receive them:
uint8 E4M3 bytes, uint16 bfloat16 bit patterns, packed uint8 E2M1 nibbles,
int8 codes, float32 scales.
"""

from __future__ import annotations

import numpy as np

from .formats import (
    E4M3_MAX,
    bf16_bits_to_f64,
    e2m1_to_f64,
    e4m3_to_f64,
    f64_to_e4m3_codes,
    unpack_nibbles,
)

__all__ = [
    "fp8_materialize",
    "fp8_linear",
    "fp8_grouped",
    "nvfp4_dequant",
    "nvfp4_linear",
    "int8_quantize_act",
    "int8_accumulate",
    "int8_epilogue",
    "int8_grouped",
    "fp8_quantize_act",
    "fp8_w8a8_linear",
    "bf16_linear",
    "ACTIVATIONS",
    "activation",
    "apply_epilogue",
]

_ROW_CHUNK = 8192  # weight rows decoded to float64 at a time (bounds memory on the widest layer)


def fp8_materialize(w_codes) -> np.ndarray:
    """FP8 weight -> dense [N, K] values (fp8_gemv page, ``enqueue_fp8_materialize``)."""
    return e4m3_to_f64(w_codes)


def _linear(decode_rows, n_rows: int, x_bits, alpha: float):
    """out[m, n] = alpha * sum_k x[m,k] * Wdec[n,k] in float64, plus the bound
    B[m, n] = |alpha| * sum_k |x[m,k] * Wdec[n,k]|.  ``decode_rows(lo, hi)``
    returns the decoded float64 weight rows lo..hi-1."""
    x = bf16_bits_to_f64(x_bits)
    if x.ndim != 2:
        raise ValueError("activation must be [M, K]")
    m = x.shape[0]
    ref = np.empty((m, n_rows), dtype=np.float64)
    bound = np.empty((m, n_rows), dtype=np.float64)
    ax = np.abs(x)
    for lo in range(0, n_rows, _ROW_CHUNK):
        hi = min(n_rows, lo + _ROW_CHUNK)
        w = decode_rows(lo, hi)
        ref[:, lo:hi] = x @ w.T
        bound[:, lo:hi] = ax @ np.abs(w).T
    return alpha * ref, abs(alpha) * bound


def fp8_linear(w_codes, x_bits, alpha: float = 1.0):
    """W8A16 linear: out = alpha * x @ dec8(W)^T.

    fp8_gemv page, summary ("out = x @ dequant(W)^T") and "Scale contract"
    (the kernel returns the raw product; the per-tensor weight_scale is a
    scalar that multiplies the raw result).  ``alpha = 1`` is the raw result.
    w_codes: uint8 [N, K]; x_bits: uint16 [M, K].  Returns (ref, bound), both
    float64 [M, N].
    """
    w = np.asarray(w_codes, dtype=np.uint8)
    if w.ndim != 2:
        raise ValueError("weight must be [N, K]")
    x = np.asarray(x_bits, dtype=np.uint16)
    if x.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    return _linear(lambda lo, hi: e4m3_to_f64(w[lo:hi]), w.shape[0], x, alpha)


def _grouped(linear_of_expert, e_count: int, n: int, x_bits, a_offsets, expert_ids):
    """The ragged group loop shared by the grouped readings below: group z
    covers rows a_offsets[z] .. a_offsets[z+1]-1 (clipped to T; empty when the
    end does not exceed the start) and uses expert expert_ids[z]; an id outside
    0..E-1 writes zeros; rows no group covers stay NaN with written[r] = False.
    linear_of_expert(e, x_rows) returns (ref, bound) for one expert; x_rows
    are rows start .. end-1 of x_bits, passed as stored."""
    x = np.asarray(x_bits)
    offs = np.asarray(a_offsets).astype(np.int64)
    ids = np.asarray(expert_ids).astype(np.int64)
    t = x.shape[0]
    if offs.shape[0] != ids.shape[0] + 1:
        raise ValueError("a_offsets must have one entry more than expert_ids")
    ref = np.full((t, n), np.nan)
    bound = np.full((t, n), np.nan)
    written = np.zeros(t, dtype=bool)
    for z in range(ids.shape[0]):
        start = min(int(offs[z]), t)
        end = min(int(offs[z + 1]), t)
        if end <= start:
            continue
        e = int(ids[z])
        if 0 <= e < e_count:
            r, b = linear_of_expert(e, x[start:end])
        else:
            r = np.zeros((end - start, n))
            b = np.zeros((end - start, n))
        ref[start:end] = r
        bound[start:end] = b
        written[start:end] = True
    return ref, bound, written


def fp8_grouped(w_codes, x_bits, a_offsets, expert_ids, expert_scale=None):
    """Grouped (MoE) W8A16 linear.

    Matmul2dFp8 page, ``run_grouped``: group z covers the activation rows
    a_offsets[z] .. a_offsets[z+1]-1 and multiplies them by the transposed
    weight of expert expert_ids[z]; an inactive group (id -1) writes zeros for
    its rows; an empty group writes nothing.  The result is raw (no scale).

    Readings where the page is silent: a_offsets has one more entry than
    expert_ids; rows that no group covers are left untouched (returned as NaN
    here, with written[r] = False); an id outside 0..E-1 behaves as -1; a
    group whose end does not exceed its start is empty; row indices are
    clipped to the T activation rows.

    w_codes: uint8 [E, N, K]; x_bits: uint16 [T, K]; a_offsets: [G+1];
    expert_ids: [G].  ``expert_scale`` ([E] or None): the per-expert
    weight_scale that the page leaves to the graph as a post-matmul multiply,
    folded here as the alpha of the expert's rows (fp8_linear's scale fold).
    Returns (ref [T, N], bound [T, N], written [T]).
    """
    w = np.asarray(w_codes, dtype=np.uint8)
    e_count, n, _ = w.shape
    sc = (lambda e: 1.0) if expert_scale is None else (lambda e: float(np.float32(expert_scale[e])))
    return _grouped(lambda e, xr: fp8_linear(w[e], xr, sc(e)), e_count, n, x_bits, a_offsets, expert_ids)


def nvfp4_grouped(w_packed, w_scale_codes, x_bits, a_offsets, expert_ids, expert_scale=None):
    """Grouped (MoE) W4A16 NVFP4 linear: the ``run_grouped`` addressing of the
    Matmul2dFp8 page applied to the fp4_matmul page's weight format.

    Same group readings as fp8_grouped; expert e's weight is the NVFP4 pair
    (w_packed[e] uint8 [N, K/2], w_scale_codes[e] E4M3 [N, K/16]).  The result
    is raw: each expert's per-tensor global scale (weight_scale_2) is left to
    the caller, as the per-expert FP8 weight_scale is for fp8_grouped, unless
    ``expert_scale`` ([E]) is given: then it is expert e's alpha.
    Returns (ref [T, N], bound [T, N], written [T]).
    """
    p = np.asarray(w_packed, dtype=np.uint8)
    sc = np.asarray(w_scale_codes, dtype=np.uint8)
    e_count, n, _ = p.shape
    es = (lambda e: 1.0) if expert_scale is None else (lambda e: float(np.float32(expert_scale[e])))
    return _grouped(lambda e, xr: nvfp4_linear(p[e], sc[e], xr, es(e)), e_count, n, x_bits, a_offsets,
                    expert_ids)


def nvfp4_dequant(w_packed, w_scale_codes) -> np.ndarray:
    """NVFP4 weight -> dense values D[n, k] = e2m1(code(n, k)) * e4m3(S[n, k // 16]).

    fp4_matmul page, summary: packed ``uint8 [N, K//2]`` lo-nibble-first codes
    and ``float8_e4m3fn [N, K//16]`` block scales, one scale per 16
    consecutive k of a row.  Returns float64 [N, K].
    """
    p = np.asarray(w_packed, dtype=np.uint8)
    s = np.asarray(w_scale_codes, dtype=np.uint8)
    n, half_k = p.shape
    k = 2 * half_k
    if k % 16 != 0 or s.shape != (n, k // 16):
        raise ValueError("block scales must be [N, K//16] with K % 16 == 0")
    codes = unpack_nibbles(p)
    block_of_k = np.arange(k) // 16
    return e2m1_to_f64(codes) * e4m3_to_f64(s)[:, block_of_k]


def nvfp4_linear(w_packed, w_scale_codes, x_bits, alpha: float = 1.0):
    """W4A16 NVFP4 linear: out = alpha * x @ D^T with D from ``nvfp4_dequant``.

    fp4_matmul page, summary (``out = activation @ weight^T``,
    ``enqueue_apple_fp4_matmul``); alpha is the per-tensor global scale
    (weight_scale_2, fp8_gemv page "Scale contract").  Returns (ref, bound).
    """
    p = np.asarray(w_packed, dtype=np.uint8)
    s = np.asarray(w_scale_codes, dtype=np.uint8)
    return _linear(lambda lo, hi: nvfp4_dequant(p[lo:hi], s[lo:hi]), p.shape[0], x_bits, alpha)


def int8_quantize_act(x_bits):
    """Per-row symmetric absmax int8 quantisation of a bfloat16 activation.

    int8_matmul page, "Quantization (W8A8)": scale = absmax / 127 per row;
    ``AppleInt8ActQuant`` / ``enqueue_apple_int8_quantize_activation``:
    (M, K) -> int8 q + fp32 a_scale (M,).

    Readings where the page is silent, all in float32 (the precision of the
    returned scale): absmax = max_k |x[m,k]| (exact); a_scale = absmax / 127
    with one IEEE float32 division; q = round-half-even(x / a_scale) with one
    IEEE float32 division, clamped to [-127, 127]; an all-zero row gets
    a_scale = 0 and q = 0.  Non-finite inputs (outside the page's workloads)
    follow the same formulas: a NaN makes the row's absmax and a_scale NaN,
    an infinity makes them +inf; such a row's codes are all 0 (every
    quotient is then NaN or 0), so its dequantised outputs are NaN.
    """
    x = bf16_bits_to_f64(x_bits).astype(np.float32)   # exact widening
    if x.ndim != 2:
        raise ValueError("activation must be [M, K]")
    absmax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    a_scale = np.divide(absmax, np.float32(127.0), dtype=np.float32)
    q = np.zeros(x.shape, dtype=np.int8)
    rows = (a_scale > 0) & np.isfinite(a_scale)
    if np.any(rows):
        ratio = np.divide(x[rows], a_scale[rows, None], dtype=np.float32)
        q[rows] = np.clip(np.rint(ratio), -127, 127).astype(np.int8)
    return q, a_scale.astype(np.float32)


def int8_accumulate(a_codes, b_codes) -> np.ndarray:
    """int32 accumulators acc[m, n] = sum_k a[m,k] * b[n,k] (int8_matmul page,
    summary: ``out = dequant(A_int8 @ B_int8^T)``, accumulation in int32).

    Evaluated as a float64 BLAS product of the int8 values: every product and
    every partial sum is an integer of magnitude <= K * 127^2, exact in
    float64 for K < 2^53 / 127^2, so the result is exact in any order.
    Returns int64 [M, N].
    """
    a = np.asarray(a_codes, dtype=np.int8).astype(np.float64)
    b = np.asarray(b_codes, dtype=np.int8).astype(np.float64)
    if a.shape[1] * 127 * 127 >= 2 ** 53:
        raise ValueError("K too large for an exact float64 accumulation")
    return (a @ b.T).astype(np.int64)


def int8_epilogue(acc, a_scale, b_scale, bias_bits=None):
    """Dequantise int32 accumulators: out = acc * a_scale[m] * b_scale[n] + bias[n].

    int8_matmul page, "Quantization (W8A8)": each output is dequantised by
    a_scale[row] * b_scale[col] and the optional per-column bias is added after
    the dequantisation.  Reading: bias is bfloat16 [N]; the float64 result is
    rounded once by the caller.  Returns (ref float64 [M, N], tau float64 [M, N])
    where tau = 2^-22 * (|acc * a_s * b_s| + |bias|) + 1e-6 is the float32
    evaluation slack of the epilogue (four float32 roundings at most).
    """
    acc = np.asarray(acc, dtype=np.float64)
    a_s = np.asarray(a_scale, dtype=np.float32).astype(np.float64)
    b_s = np.asarray(b_scale, dtype=np.float32).astype(np.float64)
    with np.errstate(invalid="ignore"):   # 0 * inf: a row whose a_scale is not finite gives NaN
        prod = acc * a_s[:, None] * b_s[None, :]
    if bias_bits is None:
        bias = np.zeros(acc.shape[1])
    else:
        bias = bf16_bits_to_f64(bias_bits)
    ref = prod + bias[None, :]
    tau = 2.0 ** -22 * (np.abs(prod) + np.abs(bias)[None, :]) + 1e-6
    return ref, tau


def int8_grouped(a_codes, b_codes, a_scale, b_scale, bias_bits, a_offsets, expert_ids, raw: bool = False):
    """Grouped (MoE) W8A8 int8: the ``run_grouped`` addressing of the
    Matmul2dFp8 page applied to the int8_matmul page's body.

    Group z covers activation rows a_offsets[z] .. a_offsets[z+1]-1 (already
    quantised per row: a_codes int8 [T, K], a_scale float32 [T]) and expert
    e = expert_ids[z] (b_codes int8 [E, N, K], b_scale float32 [E, N], bias
    bfloat16 bits [E, N] or None): acc = int8_accumulate, out = int8_epilogue
    with that expert's b_scale and bias.  Group readings as fp8_grouped.
    raw=True returns the exact accumulators instead (inactive rows 0).
    Returns (ref [T, N], tau [T, N], written [T]); tau as int8_epilogue's
    (0 for raw and for inactive rows).
    """
    a = np.asarray(a_codes, dtype=np.int8)
    b = np.asarray(b_codes, dtype=np.int8)
    a_s = np.asarray(a_scale, dtype=np.float32)
    b_s = np.asarray(b_scale, dtype=np.float32)
    e_count, n, _ = b.shape
    bias = None if bias_bits is None else np.asarray(bias_bits, dtype=np.uint16)

    def expert(e, rows):
        acc = int8_accumulate(a[rows], b[e])
        if raw:
            return acc.astype(np.float64), np.zeros(acc.shape)
        return int8_epilogue(acc, a_s[rows], b_s[e], None if bias is None else bias[e])

    return _grouped(expert, e_count, n, np.arange(a.shape[0]), a_offsets, expert_ids)


def fp8_quantize_act(x_bits, input_scale: float) -> np.ndarray:
    """Static per-tensor FP8 quantisation of a bfloat16 activation (W8A8).

    fp8_gemv page, "Scale contract": the per-tensor ``input_scale`` of a
    modelopt FP8 checkpoint cancels only while the activation stays bf16; for
    fp8 activations it is the quantisation step.  Readings (the page gives no
    formula): q = E4M3(clamp(x / input_scale, -448, 448)), the division one IEEE
    float32 division and the rounding to nearest, ties to even, in one step from
    that float32 quotient; input_scale > 0.  Returns uint8 E4M3 codes [M, K].
    """
    x = bf16_bits_to_f64(x_bits).astype(np.float32)             # exact widening
    s = np.float32(input_scale)
    if not s > 0:
        raise ValueError("input_scale must be positive")
    with np.errstate(over="ignore"):      # quotients beyond float32 saturate at the clamp
        v = np.divide(x, s, dtype=np.float32)
    v = np.clip(v, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return f64_to_e4m3_codes(v.astype(np.float64))


def fp8_w8a8_linear(xq_codes, w_codes, alpha: float = 1.0):
    """FP8 W8A8 linear: out = alpha * dec(xq) @ dec(W)^T, both operands E4M3.

    The fp8_gemv page's weight and layout with fp8 activations: alpha is
    input_scale * weight_scale, applied once to the float64 sum.  Every product
    of two E4M3 values is exact.  Returns (ref [M, N], bound [M, N]).
    """
    x = e4m3_to_f64(xq_codes)
    if x.ndim != 2:
        raise ValueError("activation must be [M, K]")
    w = np.asarray(w_codes, dtype=np.uint8)
    m, n_rows = x.shape[0], w.shape[0]
    ref = np.empty((m, n_rows), dtype=np.float64)
    bound = np.empty((m, n_rows), dtype=np.float64)
    ax = np.abs(x)
    for lo in range(0, n_rows, _ROW_CHUNK):
        hi = min(n_rows, lo + _ROW_CHUNK)
        wd = e4m3_to_f64(w[lo:hi])
        ref[:, lo:hi] = x @ wd.T
        bound[:, lo:hi] = ax @ np.abs(wd).T
    return alpha * ref, abs(alpha) * bound


def bf16_linear(w_bits, x_bits, alpha: float = 1.0):
    """Dense control: out = alpha * x @ W^T with a bfloat16 weight [N, K].

    The comparison point the quantized paths are measured against: the bf16
    weight path of the fp8_gemv page ("WHY it wins at decode": 2 bytes per
    weight against W8A16's 1) and the dense bf16 GEMM the Matmul2dFp8 page's
    tiled kernel mirrors with only the weight type changed (summary).
    w_bits: uint16 [N, K]; x_bits: uint16 [M, K].  Returns (ref, bound),
    both float64 [M, N].
    """
    w = np.asarray(w_bits, dtype=np.uint16)
    if w.ndim != 2:
        raise ValueError("weight must be [N, K]")
    x = np.asarray(x_bits, dtype=np.uint16)
    if x.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    return _linear(lambda lo, hi: bf16_bits_to_f64(w[lo:hi]), w.shape[0], x, alpha)


ACTIVATIONS = ("none", "relu", "silu", "gelu_tanh")


def activation(v, name: str) -> np.ndarray:
    """The epilogue activations by their definitions, in float64: ReLU
    max(v, 0); SiLU v / (1 + e^-v); GELU in its tanh form
    0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715 v^3).  The GELU is
    evaluated through the identity 1 + tanh(u) = 2 / (1 + e^-2u), i.e. as
    v / (1 + e^-2u): the same function, but the literal form cancels to 0 in
    double precision once u < -19 (v below about -6), where the result is
    still a normal bfloat16 number."""
    v = np.asarray(v, dtype=np.float64)
    if name == "none":
        return v.copy()
    if name == "relu":
        return np.maximum(v, 0.0)
    if name == "silu":
        with np.errstate(over="ignore"):
            return v / (1.0 + np.exp(-v))
    if name == "gelu_tanh":
        u = np.sqrt(2.0 / np.pi) * (v + 0.044715 * v ** 3)
        with np.errstate(over="ignore"):
            return v / (1.0 + np.exp(-2.0 * u))
    raise ValueError(f"unknown activation {name!r}")


def apply_epilogue(value, row_scale=None, col_scale=None, bias_bits=None, act: str = "none", residual=None):
    """Fused epilogue on an [M, N] float64 result whose alpha is applied.

    Matmul2dFp8 page, "Parameters": elementwise_lambda_fn is an optional
    element-wise function of each output element's (row, col) coordinates and
    value, fused into the store.  Reading: a fixed menu of such steps, in this
    order -- times row_scale[m], times col_scale[n], plus bias[n] (bfloat16
    bits), the activation, plus residual[m, n] -- following the int8_matmul
    page's epilogue, which scales first and adds the per-column bias after.
    Missing steps (None, "none") are skipped.  ``residual`` holds values
    (float64-convertible), already decoded.

    Returns (out, parts): ``parts`` carries the intermediate magnitudes the
    acceptance rule of ``oracle.compare.epilogue_tolerance`` needs: "scale"
    |row_scale[m] col_scale[n]|, "scaled" the value after the scales, "pre" the
    activation's input, "post" its output, "residual" |residual| and "out".
    """
    v = np.asarray(value, dtype=np.float64)
    m, n = v.shape
    scale = np.ones((m, n))
    if row_scale is not None:
        rs = np.asarray(row_scale, dtype=np.float64).reshape(m, 1)
        v = v * rs
        scale = scale * np.abs(rs)
    if col_scale is not None:
        cs = np.asarray(col_scale, dtype=np.float64).reshape(1, n)
        v = v * cs
        scale = scale * np.abs(cs)
    scaled = v
    if bias_bits is not None:
        v = v + bf16_bits_to_f64(np.asarray(bias_bits, dtype=np.uint16)).reshape(1, n)
    pre = v
    post = activation(pre, act)
    out = post
    res = np.zeros((m, n))
    if residual is not None:
        res = np.asarray(residual, dtype=np.float64).reshape(m, n)
        out = post + res
    parts = {"scale": scale, "scaled": scaled, "pre": pre, "post": post, "residual": np.abs(res), "out": out}
    return out, parts
