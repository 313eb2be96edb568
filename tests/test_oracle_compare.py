"""Pins of the acceptance rules (oracle.compare): they accept what they must
and reject plausible mistakes."""

import numpy as np

from oracle import compare as C
from oracle import formats as F


def test_bf16_ordered_and_ulp():
    b = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3F80, 0x3F81, 0x7F7F], np.uint16)
    o = C.bf16_ordered(b)
    assert o[0] == o[1] == 0 and o[2] == 1 and o[3] == -1 and o[5] - o[4] == 1
    u = C.bf16_ulp(np.array([0x3F80, 0x4000, 0x0000, 0x0080], np.uint16))
    assert list(u) == [2.0 ** -7, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133]


def test_check_bf16_accepts_neighbours_rejects_two_ulps():
    ref = np.array([1.0 + 2.0 ** -9, 3.0, -5.25, 0.0])
    r = F.f64_to_bf16_bits(ref)
    tau = np.zeros(4)
    assert C.check_bf16(r, ref, tau)
    def step(bits, d):
        # move d places along the ordered bf16 line
        o = C.bf16_ordered(bits) + d
        return np.where(o < 0, 0x8000 | (-o), o).astype(np.uint16)
    assert C.check_bf16(step(r, 1), ref, tau)
    assert C.check_bf16(step(r, -1), ref, tau)
    assert not C.check_bf16(step(r, -2), ref, tau)
    bad = r.copy()
    bad[1] += 2
    res = C.check_bf16(bad, ref, tau)
    assert not res and res.n_bad == 1
    # +0 vs -0 are equal
    assert C.check_bf16(np.array([0x8000], np.uint16), np.array([0.0]), np.zeros(1))


def test_check_bf16_clause2_cancellation():
    ref = np.array([1e-6])
    gpu = F.f64_to_bf16_bits(np.array([3e-6]))      # many bf16 ulps away but within tau
    assert C.check_bf16(gpu, ref, np.array([5e-6])).n_clause2 == 1
    assert not C.check_bf16(gpu, ref, np.array([1e-7]))


def test_check_f32_bound_and_nan():
    ref = np.array([1.0, 2.0, np.nan])
    b = np.array([100.0, 100.0, 1.0])
    assert C.check_f32(np.array([1.1, 1.9, np.nan], np.float32), ref, b)
    assert not C.check_f32(np.array([1.3, 2.0, np.nan], np.float32), ref, b)
    assert not C.check_f32(np.array([1.0, 2.0, 0.0], np.float32), ref, b)
    assert not C.check_f32(np.array([np.nan, 2.0, np.nan], np.float32), ref, b)


def test_tolerance_rejects_a_dropped_row_of_terms():
    """A kernel that drops every product of one K-chunk (1/16 of the terms)
    must fail the rule on realistic data."""
    r = np.random.default_rng(0)
    k = 4096
    x = r.standard_normal((1, k))
    w = r.standard_normal((64, k)) * 0.02
    ref = x @ w.T
    bound = np.abs(x) @ np.abs(w).T
    mask = np.ones(k)
    mask[:256] = 0
    bad = (x * mask) @ w.T
    assert not C.check_f32(bad.astype(np.float32), ref, bound)
