"""Pins for the NVFP4 oracle: the E2M1 grid and its rounding against brute force, the
per-matrix scale's bounds, the MSE scale choice against an exhaustive float64 search,
exact round trips, and the packing order."""
import numpy as np
import pytest

from oracle import nvfp4 as NV
from oracle import mxfp8 as MX


def test_e2m1_values_and_codes():
    assert list(NV.e2m1_decode(np.arange(8))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(NV.e2m1_decode(np.arange(8, 16))) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    for c in range(16):                                  # every code round-trips
        assert NV.e2m1_encode(np.float32(NV.e2m1_decode(c))) == c or (c == 8 and NV.e2m1_encode(np.float32(-0.0)) == 8)


def test_e2m1_rounding_against_brute_force():
    x = np.concatenate([np.linspace(-8, 8, 4097), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 1e-9, 7e5]])
    x = x.astype(np.float32)
    got = NV.e2m1_decode(NV.e2m1_encode(x))
    mags = NV.E2M1_VALUES
    for xi, gi in zip(x, got):
        a = min(abs(float(xi)), 6.0)
        d = np.abs(mags - a)
        best = np.nonzero(d == d.min())[0]
        want = mags[best[0]] if len(best) == 1 else mags[[b for b in best if b % 2 == 0][0]]  # tie: even code
        assert abs(gi) == want, (xi, gi, want)
        assert np.signbit(gi) == np.signbit(xi) or gi == 0


def test_global_scale_is_tight_power_of_two():
    rng = np.random.default_rng(1)
    for scale in (1e-6, 0.02, 1.0, 3e3):
        w = (rng.standard_normal((8, 64)) * scale).astype(np.float32)
        g = float(NV.global_scale(w))
        assert np.log2(g) == np.round(np.log2(g))
        need = np.abs(w).max() / 6.0 / g
        assert 224.0 < need <= 448.0
    assert NV.global_scale(np.zeros((2, 16))) == 1.0


def test_scale_choice_is_the_float64_minimum():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((4, 16 * 6)) * 0.02).astype(np.float32)
    w[0, :16] = 0.0                                      # all-zero block: smallest code
    w[1, 16:32] = w[1, 16]                               # constant block
    packed, scales, g = NV.quantize(w)
    assert scales[0, 0] == 1
    for r in range(4):
        for b in range(6):
            blk = w[r, 16 * b:16 * b + 16]
            errs = NV.block_errors_f64(blk, float(g))
            chosen = errs[int(scales[r, b]) - 1]
            assert chosen <= errs.min() * (1 + 1e-5) + 1e-30, (r, b)
            # at least as good as maximum scaling (the E4M3 code nearest amax / 6 / g)
            mx = int(MX.e4m3_encode(np.abs(blk).max() / 6.0 / float(g)))
            if mx > 0:
                assert chosen <= errs[mx - 1] * (1 + 1e-6) + 1e-30


def test_exact_round_trip_and_packing():
    rng = np.random.default_rng(3)
    g = 2.0 ** -10
    codes = rng.integers(0, 16, size=(3, 32))
    sc = rng.integers(0x30, 0x50, size=(3, 2))
    w = NV.e2m1_decode(codes) * np.repeat(MX.e4m3_decode(sc), 16, axis=1) * g
    w[:, 0] = 6.0 * MX.e4m3_decode(sc[:, 0]) * g          # pin each block's amax to a grid point
    packed, scales, gq = NV.quantize(w.astype(np.float32))
    back = NV.dequantize(packed, scales, gq)
    np.testing.assert_array_equal(back, w)               # error 0 is the minimum: exact
    # packing: element 2j in the low nibble of byte j
    one = np.zeros((1, 16), dtype=np.float32)
    one[0, 2] = 6.0 * 2.0 ** -3
    p, s, g1 = NV.quantize(one)
    assert p[0, 1] & 15 == 7 and p[0, 1] >> 4 == 0 and np.all(p[0, [0, 2, 3]] == 0)


def test_dequantised_values_are_bf16_exact():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((16, 128)) * 0.02).astype(np.float32)
    d = NV.dequantize(*NV.quantize(w))
    bits = d.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)                    # bfloat16 keeps the upper 16 bits
    assert np.all(d.astype(np.float32) == d)
    # and the format's error: relative RMS well below 2^-2 per block
    assert np.sqrt(np.mean((d - w) ** 2)) < 0.15 * np.sqrt(np.mean(w.astype(np.float64) ** 2))
