"""Pins of the oracle's format decoders (oracle.formats) against things other
than themselves: hand-worked codes (tests/golden), torch's own float8 and
bfloat16 conversions, closed forms and invariants."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import formats as F


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(s):
    return float("nan") if s == "nan" else float(s)


# ------------------------------------------------------------------ E4M3

def test_e4m3_golden_codes():
    g = _load("e4m3_codes.json")
    for e in g["entries"]:
        code = int(e["code"], 16)
        got = F.e4m3_to_f64(np.array([code], np.uint8))[0]
        want = _num(e["value"])
        if np.isnan(want):
            assert np.isnan(got), e
        else:
            assert got == want and np.signbit(got) == np.signbit(want), (e, got)


def test_e4m3_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    fin = ~np.isnan(ours)
    assert np.array_equal(ours[fin], lib[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(lib[fin]))


def test_e4m3_closed_forms():
    g = _load("e4m3_codes.json")["closed_forms"]
    v = F.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert int(np.sum(np.isfinite(v))) == g["finite_code_count"]
    assert set(np.flatnonzero(np.isnan(v)).tolist()) == {0x7F, 0xFF}
    pos = v[:128][np.isfinite(v[:128])]
    assert sum(Fraction(float(t)) for t in pos) == Fraction(g["sum_of_non_negative_finite_values"])
    # strictly increasing over the non-negative codes; sign symmetry
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(v[128:][np.isfinite(v[128:])], -pos)
    assert np.nanmax(np.abs(v)) == 448.0


def test_e4m3_each_value_exact_in_bf16_and_products_exact_in_f32():
    """Every finite E4M3 value has <= 4 significant bits, so it is a bfloat16
    and its product with any bfloat16 is exact in float32 (checked by brute
    force over all bf16 mantissas at exponent 0 and the full E4M3 range)."""
    v = F.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    v = v[np.isfinite(v)]
    assert np.array_equal(F.bf16_bits_to_f64(F.f64_to_bf16_bits(v)), v)
    mant = F.bf16_bits_to_f64(np.arange(0x3F80, 0x4000, dtype=np.uint16))  # [1, 2)
    prod = np.outer(mant, v)
    assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)


# ------------------------------------------------------------------ E2M1 / nibbles

def test_e2m1_golden_table():
    g = _load("e2m1_nibbles.json")
    got = F.e2m1_to_f64(np.arange(16))
    for c, s in g["codes"].items():
        w = float(s)
        assert got[int(c)] == w and np.signbit(got[int(c)]) == np.signbit(w)
    assert got[:8].sum() == float(g["sum_of_positive_magnitudes"])


def test_nibble_order_golden():
    g = _load("e2m1_nibbles.json")
    for e in g["packed_bytes"]:
        codes = F.unpack_nibbles(np.array([[int(e["byte"], 16)]], np.uint8))
        vals = F.e2m1_to_f64(codes)[0]
        assert vals[0] == float(e["k_even"]) and vals[1] == float(e["k_odd"]), e


def test_e2m1_rejects_wide_codes():
    with pytest.raises(ValueError):
        F.e2m1_to_f64(np.array([16]))


def test_nvfp4_products_exact_in_bf16():
    """All 16 x 254 products of an E2M1 value and a finite E4M3 scale are
    exact in bfloat16 (<= 5 significant bits, range [2^-10, 2688])."""
    e2 = F.e2m1_to_f64(np.arange(16))
    e4 = F.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    e4 = e4[np.isfinite(e4)]
    p = np.outer(e2, e4).ravel()
    assert np.array_equal(F.bf16_bits_to_f64(F.f64_to_bf16_bits(p)), p)
    nz = np.abs(p[p != 0])
    assert nz.min() == 2.0 ** -10 and nz.max() == 2688.0


# ------------------------------------------------------------------ bfloat16

def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = F.bf16_bits_to_f64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


def test_bf16_round_matches_torch_on_float32_inputs():
    """For inputs that are float32, one rounding float64 -> bf16 equals
    torch's float32 -> bf16 cast (RNE).  Covers random values, exact ties,
    subnormals and the overflow boundary."""
    r = np.random.default_rng(7)
    x = r.standard_normal(200000).astype(np.float32) * np.float32(1e3)
    ties = (F.bf16_bits_to_f64(r.integers(0, 0x7F7F, 5000).astype(np.uint16)) *
            (1 + 2.0 ** -8)).astype(np.float32)           # halfway between two bf16 values
    sub = (r.standard_normal(5000) * 1e-39).astype(np.float32)
    edge = np.array([3.3895313e38, 3.3961775e38, 3.4e38, -3.4e38, 1e-45, -0.0, 0.0], np.float32)
    allx = np.concatenate([x, ties, sub, edge])
    ours = F.f64_to_bf16_bits(allx.astype(np.float64))
    lib = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


def test_bf16_round_is_single_rounding_from_f64():
    """1 + 2^-8 + 2^-30 rounds directly to 1 + 2^-7; going through float32
    first would give the tie 1 + 2^-8 and then 1.0."""
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.bf16_bits_to_f64(F.f64_to_bf16_bits(np.array([v])))[0] == 1.0 + 2.0 ** -7
    # exact ties go to the even mantissa
    t = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)])
    assert list(F.bf16_bits_to_f64(F.f64_to_bf16_bits(t))) == [1.0, 1 + 2.0 ** -6, -1.0]
    assert F.f64_to_bf16_bits(np.array([np.nan]))[0] & 0x7FFF == 0x7FC0


def test_round_to_precision_brute_force():
    """Compare with an exact-rational nearest search on a small grid."""
    p, emin = 4, -3
    grid = set()
    for e in range(emin, 4):
        for m in range(2 ** (p - 1), 2 ** p):
            grid.add(Fraction(m, 2 ** (p - 1)) * Fraction(2) ** e)
    for m in range(0, 2 ** (p - 1)):
        grid.add(Fraction(m, 2 ** (p - 1)) * Fraction(2) ** emin)
    grid = sorted(grid)
    xs = np.linspace(0, 15, 4001)
    got = F.round_to_precision(xs, p, emin)
    for x, g in zip(xs, got):
        fx = Fraction(float(x))
        best = min(grid, key=lambda q: (abs(q - fx), 0))
        cands = [q for q in grid if abs(q - fx) == abs(best - fx)]
        if len(cands) == 2:  # tie: even last mantissa bit
            def even(q):
                e = emin
                while q >= Fraction(2) ** (e + 1) and e < 3:
                    e += 1
                return (q / Fraction(2) ** (e - p + 1)).numerator % 2 == 0
            best = [q for q in cands if even(q)][0]
        assert Fraction(float(g)) == best, (x, g, best)
