"""Seeded generators for the five workloads of the quantized linear layer.

Recipes (all draws from ``numpy.random.default_rng(SeedSequence(key))``):

* FP8 weights: W ~ N(0, 0.02^2) in float32, per-tensor scale
  s = float32(max|W| / 448), codes = float8_e4m3fn(clamp(W / s, +-448)) with
  round-to-nearest-even (torch's cast; the clamp keeps torch from overflowing
  to NaN).  The scale s is the checkpoint's weight_scale.
* Activations: float32 N(0, 1) rounded to bfloat16 (torch's cast, RNE).  The
  int8 workload multiplies a Bernoulli(0.01) subset by 20 before rounding.
* NVFP4 weights: W ~ N(0, 0.02^2); global g = float32(max|W| / (448 * 6));
  per-16 block scale S = float8_e4m3fn(clamp(block_absmax / 6 / g, 448));
  codes = E2M1 round-to-nearest-even of W / (S * g), saturating at +-6, ties to
  the even code; a zero block scale gives zero codes.  Packed two per byte,
  the even k in the low nibble.  alpha = g.
* int8 weights: per output row n, b_scale[n] = float32(max_k |W[n,k]| / 127),
  b = clamp(rint(W / b_scale), +-127); bias = bfloat16 N(0, 1).
* Grouped routing: 64 groups, group z has Zipf rank z+1 (p_r ~ r^-1.2),
  counts ~ Multinomial(T, p); the three smallest groups are emptied and their
  tokens moved to the largest; the two non-empty groups whose counts are
  nearest the median of the non-empty counts get expert id -1; the other ids
  come from a permutation of the 64 experts drawn after the multinomial.

"Dyadic" variants draw operands whose every product and partial sum is exact
in float32, so a GPU result must equal the reference bit for bit.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "rng_for",
    "bf16_bits_from_f32",
    "f32_from_bf16_bits_torch",
    "e4m3_codes_from_f32",
    "e4m3_values_torch",
    "e2m1_codes_from_f64",
    "pack_nibbles",
    "fp8_weight",
    "bf16_activation",
    "nvfp4_weight",
    "int8_weight",
    "bf16_bias",
    "grouped_routing",
    "dyadic_fp8_weight",
    "dyadic_activation",
    "dyadic_nvfp4_weight",
    "Fp8Case",
    "Nvfp4Case",
    "GroupedCase",
    "GroupedNvfp4Case",
    "Int8Case",
    "CONFIG2_SHAPES",
    "CONFIG2_M",
    "config1_case",
    "config2_case",
    "config3_case",
    "config4_case",
    "config5_case",
    "grouped_nvfp4_case",
    "bf16_weight",
    "dyadic_bf16_weight",
    "GroupedInt8Case",
    "grouped_int8_case",
    "Fp8W8A8Case",
    "fp8_w8a8_case",
    "dyadic_e4m3_activation",
]


def rng_for(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


# ---------------------------------------------------------------- format stores (torch casts)

def bf16_bits_from_f32(a) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16), torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def f32_from_bf16_bits_torch(bits) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float32).numpy()


def e4m3_codes_from_f32(a) -> np.ndarray:
    """float32 -> float8_e4m3fn codes, saturating at +-448, RNE (torch's cast)."""
    a = np.clip(np.asarray(a, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def e4m3_values_torch(codes) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float32).numpy()


_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_codes_from_f64(v) -> np.ndarray:
    """Round to the nearest E2M1 value, ties to the even code, saturating at 6.
    Returns codes 0..15 (bit 3 = sign) as uint8."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.minimum(np.abs(v), 6.0)
    lo = np.clip(np.searchsorted(_E2M1_GRID, mag, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo = mag - _E2M1_GRID[lo]
    d_hi = _E2M1_GRID[hi] - mag
    take_hi = (hi != lo) & ((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    sign = (np.signbit(v) & (code != 0)).astype(np.uint8) << 3
    return code | sign


def pack_nibbles(codes) -> np.ndarray:
    """[..., K] 4-bit codes -> [..., K//2] bytes, even k in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


# ---------------------------------------------------------------- tensors

def fp8_weight(key, n: int, k: int):
    """E4M3 codes [N, K] of N(0, 0.02^2) with a per-tensor absmax/448 scale.
    Returns (codes uint8 [N, K], weight_scale float32)."""
    r = rng_for(*key)
    w = r.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    s = np.float32(np.max(np.abs(w)) / np.float32(448.0))
    codes = e4m3_codes_from_f32(w / s)
    return codes, s


def bf16_activation(key, m: int, k: int, outlier_p: float = 0.0, outlier_mul: float = 20.0):
    """bfloat16 bits [M, K] of N(0, 1), optionally with Bernoulli outliers."""
    r = rng_for(*key)
    x = r.standard_normal((m, k), dtype=np.float32)
    if outlier_p > 0:
        mask = r.random((m, k)) < outlier_p
        x = np.where(mask, x * np.float32(outlier_mul), x)
    return bf16_bits_from_f32(x)


def nvfp4_weight(key, n: int, k: int):
    """NVFP4 weight of N(0, 0.02^2).  Returns (packed uint8 [N, K//2],
    block scale codes uint8 [N, K//16], global scale g float32)."""
    if k % 16:
        raise ValueError("K must be a multiple of 16")
    r = rng_for(*key)
    w = (r.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    g = np.float32(np.max(np.abs(w)) / np.float32(448.0 * 6.0))
    blocks = w.reshape(n, k // 16, 16)
    bmax = np.max(np.abs(blocks), axis=2)
    s_codes = e4m3_codes_from_f32(bmax / np.float32(6.0) / g)
    s_val = e4m3_values_torch(s_codes).astype(np.float64)
    denom = s_val[..., None] * np.float64(g)
    with np.errstate(divide="ignore", invalid="ignore"):
        scaled = np.where(denom > 0, blocks.astype(np.float64) / denom, 0.0)
    codes = e2m1_codes_from_f64(scaled).reshape(n, k)
    return pack_nibbles(codes), s_codes, g


def int8_weight(key, n: int, k: int):
    """int8 weight codes [N, K] with per-row (per output column) scales."""
    r = rng_for(*key)
    w = r.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    b_scale = (np.max(np.abs(w), axis=1) / np.float32(127.0)).astype(np.float32)
    safe = np.where(b_scale > 0, b_scale, np.float32(1.0))
    codes = np.clip(np.rint(w / safe[:, None]), -127, 127).astype(np.int8)
    return codes, b_scale


def bf16_bias(key, n: int):
    r = rng_for(*key)
    return bf16_bits_from_f32(r.standard_normal(n, dtype=np.float32))


def grouped_routing(key, num_experts: int = 64, tokens: int = 4096, zipf_s: float = 1.2,
                    n_empty: int = 3, n_inactive: int = 2):
    """Ragged MoE routing.  Returns (a_offsets uint32 [G+1], expert_ids int32 [G],
    counts int64 [G]) with G = num_experts."""
    r = rng_for(*key)
    ranks = np.arange(1, num_experts + 1, dtype=np.float64)
    p = ranks ** -zipf_s
    p /= p.sum()
    counts = r.multinomial(tokens, p).astype(np.int64)
    perm = r.permutation(num_experts)
    largest = int(np.argmax(counts))
    order = np.argsort(counts, kind="stable")
    empties = [int(z) for z in order if z != largest][:n_empty]
    for z in empties:
        counts[largest] += counts[z]
        counts[z] = 0
    ids = perm.astype(np.int32)
    nonempty = np.flatnonzero(counts > 0)
    med = np.median(counts[nonempty])
    near = nonempty[np.argsort(np.abs(counts[nonempty] - med), kind="stable")][:n_inactive]
    ids[near] = -1
    offs = np.zeros(num_experts + 1, dtype=np.uint32)
    offs[1:] = np.cumsum(counts).astype(np.uint32)
    return offs, ids, counts


# ---------------------------------------------------------------- exact-arithmetic variants

def dyadic_fp8_weight(key, n: int, k: int) -> np.ndarray:
    """E4M3 codes whose values are multiples of 2^-4 with magnitude <= 16."""
    allc = np.arange(256, dtype=np.uint8)
    vals = e4m3_values_torch(allc)
    ok = np.isfinite(vals) & (np.abs(vals) <= 16) & (np.mod(vals * 16, 1) == 0)
    pool = allc[ok]
    return rng_for(*key).choice(pool, size=(n, k)).astype(np.uint8)


def bf16_weight(key, n: int, k: int) -> np.ndarray:
    """bfloat16 bits [N, K] of N(0, 0.02^2): the dense control's weight."""
    w = rng_for(*key).standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    return bf16_bits_from_f32(w)


def dyadic_bf16_weight(key, n: int, k: int) -> np.ndarray:
    """bfloat16 bits of multiples of 2^-4 with magnitude <= 16 (the values of
    ``dyadic_fp8_weight``): with ``dyadic_activation`` every partial sum is
    exact in float32."""
    vals = e4m3_values_torch(dyadic_fp8_weight(key, n, k)).astype(np.float32)
    return bf16_bits_from_f32(vals)


def dyadic_activation(key, m: int, k: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    """bfloat16 bits of integers in [lo, hi]."""
    x = rng_for(*key).integers(lo, hi + 1, size=(m, k)).astype(np.float32)
    return bf16_bits_from_f32(x)


def dyadic_nvfp4_weight(key, n: int, k: int):
    """NVFP4 weight with block scales in {0.5, 1}: every decoded value is a
    multiple of 0.25 with magnitude <= 6."""
    r = rng_for(*key)
    codes = r.integers(0, 16, size=(n, k)).astype(np.uint8)
    scale_pool = e4m3_codes_from_f32(np.array([0.5, 1.0], dtype=np.float32))
    s_codes = r.choice(scale_pool, size=(n, k // 16)).astype(np.uint8)
    return pack_nibbles(codes), s_codes


# ---------------------------------------------------------------- the five workloads

@dataclass
class Fp8Case:
    name: str
    w: np.ndarray            # uint8 [N, K] E4M3 codes
    x: np.ndarray            # uint16 [M, K] bfloat16 bits
    alpha: float             # per-tensor weight_scale
    out: str                 # "f32" or "bf16"

    @property
    def shape(self):
        return self.x.shape[0], self.w.shape[0], self.w.shape[1]


@dataclass
class Nvfp4Case:
    name: str
    w_packed: np.ndarray     # uint8 [N, K//2]
    w_scale: np.ndarray      # uint8 [N, K//16] E4M3 codes
    x: np.ndarray            # uint16 [M, K]
    alpha: float             # weight_scale_2
    out: str = "bf16"


@dataclass
class GroupedCase:
    name: str
    w: np.ndarray            # uint8 [E, N, K]
    x: np.ndarray            # uint16 [T, K]
    a_offsets: np.ndarray    # uint32 [G+1]
    expert_ids: np.ndarray   # int32 [G]
    max_tokens: int
    out: str = "bf16"
    weight_scale: float = 1.0


@dataclass
class GroupedNvfp4Case:
    name: str
    packed: np.ndarray       # uint8 [E, N, K/2]
    scales: np.ndarray       # uint8 [E, N, K/16] E4M3 codes
    x: np.ndarray            # uint16 [T, K]
    a_offsets: np.ndarray    # uint32 [G+1]
    expert_ids: np.ndarray   # int32 [G]
    max_tokens: int
    global_scale: float = 1.0


@dataclass
class GroupedInt8Case:
    name: str
    x: np.ndarray            # uint16 [T, K] bfloat16 bits (quantised per row by the kernel under test)
    b: np.ndarray            # int8 [E, N, K]
    b_scale: np.ndarray      # float32 [E, N]
    bias: np.ndarray         # uint16 [E, N] bfloat16 bits
    a_offsets: np.ndarray    # uint32 [G+1]
    expert_ids: np.ndarray   # int32 [G]
    max_tokens: int


@dataclass
class Fp8W8A8Case:
    name: str
    x: np.ndarray            # uint16 [M, K] bfloat16 bits
    input_scale: float       # static per-tensor activation scale (absmax / 448)
    w: np.ndarray            # uint8 [N, K] E4M3 codes
    weight_scale: float


@dataclass
class Int8Case:
    name: str
    x: np.ndarray            # uint16 [M, K] bfloat16 activation
    b: np.ndarray            # int8 [N, K]
    b_scale: np.ndarray      # float32 [N]
    bias: np.ndarray         # uint16 [N]
    extra: dict = field(default_factory=dict)


def config1_case(case: int) -> Fp8Case:
    """FP8 W8A16 GEMV at M=1, N=2048, K=2048 (case 0) or K=2050 (case 1); fp32 raw out."""
    k = (2048, 2050)[case]
    w, s = fp8_weight((1, case, 0), 2048, k)
    x = bf16_activation((1, case, 1), 1, k)
    return Fp8Case(f"gemv_m1_n2048_k{k}", w, x, float(s), "f32")


CONFIG2_SHAPES = ((4096, 4096), (14336, 4096), (4096, 14336), (128256, 4096))
CONFIG2_M = (1, 4, 16)


def config2_case(shape_idx: int, m: int, weight=None) -> Fp8Case:
    """FP8 W8A16 decode GEMV / skinny GEMM; bf16 out, alpha = weight_scale.
    The weight depends only on the shape, so M = 1, 4, 16 share it; pass
    ``weight=(codes, scale)`` to reuse one already drawn."""
    n, k = CONFIG2_SHAPES[shape_idx]
    w, s = weight if weight is not None else fp8_weight((2, shape_idx, 0), n, k)
    x = bf16_activation((2, shape_idx, 1, m), m, k)
    return Fp8Case(f"fp8_m{m}_n{n}_k{k}", w, x, float(s), "bf16")


def config3_case(m: int, n: int = 4096, k: int = 4096, weight=None) -> Nvfp4Case:
    """W4A16 NVFP4 GEMM, M in {1, 128, 2048}, N = K = 4096."""
    packed, sc, g = weight if weight is not None else nvfp4_weight((3, 0, 0), n, k)
    x = bf16_activation((3, 0, 1, m), m, k)
    return Nvfp4Case(f"nvfp4_m{m}_n{n}_k{k}", packed, sc, x, float(g))


def config4_case(num_experts: int = 64, n: int = 1536, k: int = 2048, tokens: int = 4096) -> GroupedCase:
    """Grouped MoE W8A16: 64 experts [64, 1536, 2048], 4096 tokens, Zipf(1.2) groups."""
    w, s = fp8_weight((4, 0, 0), num_experts * n, k)
    x = bf16_activation((4, 0, 1), tokens, k)
    offs, ids, counts = grouped_routing((4, 0), num_experts, tokens)
    return GroupedCase(f"grouped_e{num_experts}_n{n}_k{k}_t{tokens}", w.reshape(num_experts, n, k), x,
                       offs, ids, int(counts.max()), weight_scale=float(s))


def grouped_nvfp4_case(num_experts: int = 64, n: int = 1536, k: int = 2048, tokens: int = 4096) -> GroupedNvfp4Case:
    """Grouped MoE W4A16 NVFP4: the grouped workload's routing, activations and
    shapes with the expert stack quantised to NVFP4 (one global scale)."""
    packed, sc, g = nvfp4_weight((6, 0, 0), num_experts * n, k)
    x = bf16_activation((4, 0, 1), tokens, k)
    offs, ids, counts = grouped_routing((4, 0), num_experts, tokens)
    return GroupedNvfp4Case(f"grouped_nvfp4_e{num_experts}_n{n}_k{k}_t{tokens}",
                            packed.reshape(num_experts, n, k // 2), sc.reshape(num_experts, n, k // 16), x,
                            offs, ids, int(counts.max()), float(g))


def grouped_int8_case(num_experts: int = 64, n: int = 1536, k: int = 2048, tokens: int = 4096) -> GroupedInt8Case:
    """Grouped MoE W8A8: the grouped workload's routing and shapes with int8
    experts (per-output-channel absmax / 127 scales of N(0, 0.02^2)), a bf16
    bias per expert and the W8A8 activation recipe (1% x20 outliers)."""
    b, b_scale = int8_weight((8, 0, 0), num_experts * n, k)
    bias = bf16_bias((8, 0, 2), num_experts * n)
    x = bf16_activation((8, 0, 1), tokens, k, outlier_p=0.01)
    offs, ids, counts = grouped_routing((4, 0), num_experts, tokens)
    return GroupedInt8Case(f"grouped_int8_e{num_experts}_n{n}_k{k}_t{tokens}", x, b.reshape(num_experts, n, k),
                           b_scale.reshape(num_experts, n), bias.reshape(num_experts, n), offs, ids, int(counts.max()))


def fp8_w8a8_case(n: int, m: int = 4096, k: int = 3072) -> Fp8W8A8Case:
    """FP8 W8A8 at the W8A8 shapes: bf16 activation N(0, 1) with 1% x20
    outliers and a static per-tensor input_scale = absmax / 448 (a calibration
    of this very tensor), E4M3 weight of N(0, 0.02^2) with its per-tensor scale."""
    x = bf16_activation((7, n, 1), m, k, outlier_p=0.01)
    xf = f32_from_bf16_bits_torch(x)
    input_scale = float(np.float32(np.max(np.abs(xf)) / np.float32(448.0)))
    w, s = fp8_weight((7, n, 0), n, k)
    return Fp8W8A8Case(f"fp8_w8a8_m{m}_n{n}_k{k}", x, input_scale, w, float(s))


def dyadic_e4m3_activation(key, m: int, k: int) -> np.ndarray:
    """E4M3 codes of integers in [-4, 4]: with ``dyadic_fp8_weight`` every
    partial sum of a W8A8 product is exact in float32 up to K = 2^18 / 64."""
    r = rng_for(*key)
    v = r.integers(-4, 5, size=(m, k)).astype(np.float32)
    return e4m3_codes_from_f32(v)


def config5_case(n: int, m: int = 4096, k: int = 3072) -> Int8Case:
    """W8A8 int8: bf16 activation with 1% x20 outliers, int8 weight, bf16 bias."""
    x = bf16_activation((5, n, 1), m, k, outlier_p=0.01)
    b, b_scale = int8_weight((5, n, 0), n, k)
    bias = bf16_bias((5, n, 2), n)
    return Int8Case(f"int8_m{m}_n{n}_k{k}", x, b, b_scale, bias)
