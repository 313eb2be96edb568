"""The seeded input generators produce what their recipes say."""

import numpy as np

import synth
from oracle import formats as F


def test_fp8_weight_recipe():
    w, s = synth.fp8_weight((1, 0, 0), 64, 256)
    v = F.e4m3_to_f64(w)
    assert np.all(np.isfinite(v)) and np.abs(v).max() == 448.0       # the absmax element maps to 448
    assert 0.02 * 3 / 448 < s < 0.02 * 8 / 448
    again, s2 = synth.fp8_weight((1, 0, 0), 64, 256)
    assert np.array_equal(w, again) and s == s2                       # seeded


def test_e4m3_encoder_saturates_and_rounds_to_even():
    vals = np.array([500.0, -1e9, 448.0, 1.0625, 1.1875, 0.0], np.float32)
    codes = synth.e4m3_codes_from_f32(vals)
    assert list(F.e4m3_to_f64(codes)) == [448.0, -448.0, 448.0, 1.0, 1.25, 0.0]


def test_e2m1_encoder_round_trip_and_ties():
    grid = F.e2m1_to_f64(np.arange(16))
    assert np.array_equal(F.e2m1_to_f64(synth.e2m1_codes_from_f64(grid)), grid)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -5.0, 100.0])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, -4.0, 6.0])
    assert np.array_equal(F.e2m1_to_f64(synth.e2m1_codes_from_f64(ties)), want)


def test_nvfp4_weight_recipe():
    p, s, g = synth.nvfp4_weight((3, 9, 0), 32, 128)
    assert p.shape == (32, 64) and s.shape == (32, 8)
    sv = F.e4m3_to_f64(s)
    assert np.all(np.isfinite(sv)) and sv.max() <= 448
    codes = F.unpack_nibbles(p)
    assert np.array_equal(synth.pack_nibbles(codes), p)


def test_int8_weight_recipe():
    b, sc = synth.int8_weight((5, 1, 0), 16, 64)
    assert b.dtype == np.int8 and np.all(np.abs(b.astype(int)) <= 127)
    assert np.all(np.abs(b).max(axis=1) == 127)


def test_grouped_routing_recipe():
    offs, ids, counts = synth.grouped_routing((4, 0))
    assert offs[0] == 0 and offs[-1] == 4096 and np.all(np.diff(offs.astype(np.int64)) >= 0)
    assert (counts == 0).sum() == 3 and (ids == -1).sum() == 2
    assert np.all(counts[ids == -1] > 0)
    active = ids[(ids >= 0) & (counts > 0)]
    assert len(set(active.tolist())) == len(active) == 59


def test_dyadic_inputs_are_exact_in_float32():
    w = synth.dyadic_fp8_weight((0,), 8, 64)
    v = F.e4m3_to_f64(w)
    assert np.all(np.mod(v * 16, 1) == 0) and np.abs(v).max() <= 16
    x = F.bf16_bits_to_f64(synth.dyadic_activation((1,), 2, 64))
    assert np.all(np.mod(x, 1) == 0) and np.abs(x).max() <= 4
