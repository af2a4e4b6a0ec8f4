"""Pins for the oracle's MXFP8 (E4M3 elements, E8M0 scale per 32) encoder and decoder.

Values come from the E4M3 definition (OCP 8-bit floating point / Microscaling v1.0):
bias 7, three mantissa bits, subnormals m * 2^-9, largest finite 448, S.1111.111 NaN.
"""
import numpy as np
import pytest
import torch

from oracle import mxfp8 as M


def test_decode_table_points():
    codes = np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x39, 0x3F, 0x7E, 0xB8, 0x80])
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 1.875, 448.0, -1.0, 0.0]
    np.testing.assert_array_equal(M.e4m3_decode(codes), want)
    assert np.isnan(M.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    vals = M.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)                  # codes 0..0x7E increase strictly


def _encode_exhaustive(x):
    """Nearest finite E4M3 value by exhaustive search, ties to the even code."""
    vals = M.e4m3_decode(np.arange(0x7F))
    out = []
    for v in np.asarray(x, dtype=np.float64).ravel():
        a = min(abs(v), 448.0)
        dist = np.abs(vals - a)
        cand = np.flatnonzero(dist == dist.min())
        c = int(cand[0]) if len(cand) == 1 else int(cand[cand % 2 == 0][0])
        out.append(c | (0x80 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8).reshape(np.shape(x))


def test_encode_matches_exhaustive_search():
    vals = M.e4m3_decode(np.arange(0x7F))
    mids = (vals[1:] + vals[:-1]) / 2                 # every tie point
    rng = np.random.default_rng(7)
    x = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(0, 500, 2000), -rng.uniform(0, 500, 500),
                        rng.uniform(0, 2 ** -6, 500), [0.0, -0.0, 448.0, 464.0, 1e30]])
    np.testing.assert_array_equal(M.e4m3_encode(x), _encode_exhaustive(x))


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    np.testing.assert_array_equal(M.e4m3_encode(M.e4m3_decode(codes)), codes)


def test_encode_ties_to_even_and_saturation():
    x = np.array([1.0625, 1.1875, -1.0625, 3 * 2.0 ** -10, 2.0 ** -10, 432.0, 449.0, 1e9, -1e9])
    want = [0x38, 0x3A, 0xB8, 0x02, 0x00, 0x7E, 0x7E, 0x7E, 0xFE]
    np.testing.assert_array_equal(M.e4m3_encode(x), want)
    # just off the midpoint goes to the nearer value
    np.testing.assert_array_equal(M.e4m3_encode(np.array([1.0626, 1.0624])), [0x39, 0x38])


def test_shared_scale_rules():
    g = np.zeros((4, 32))
    g[0, 3] = 448.0 * 2.0 ** -10        # amax = 448 * 2^-10: scale 2^-10, no saturation
    g[1, 0] = -1.0                       # amax 1: scale 2^-8, element 256
    g[2, 5] = 500.0 * 2.0 ** -10         # amax in [448, 512) * 2^-10 saturates to 448
    codes, scales = M.quantize(g)        # row 3 is all zeros
    np.testing.assert_array_equal(scales[:, 0], [117, 119, 117, 0])
    assert codes[0, 3] == 0x7E and codes[1, 0] == (0x80 | M.e4m3_encode(np.array([256.0]))[0])
    assert codes[2, 5] == 0x7E
    assert np.all(codes[3] == 0)
    dq = M.dequantize(codes, scales)
    assert dq[0, 3] == g[0, 3] and dq[1, 0] == -1.0 and dq[2, 5] == 448.0 * 2.0 ** -10


def test_quantisation_error_bound_and_bf16_exactness():
    rng = np.random.default_rng(0)
    w = torch.from_numpy(rng.standard_normal((64, 256)) * 0.02).to(torch.bfloat16).double().numpy()
    codes, scales = M.quantize(w)
    dq = M.dequantize(codes, scales)
    scale = np.repeat(M.e8m0_decode(scales), 32, axis=1)
    # half a unit in the last place of the element, times the group scale
    a = np.abs(w) / scale
    ulp = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    sat = a > 448.0                     # maximum scaling leaves amax/X in [256, 512)
    assert np.all(np.abs(w - dq)[~sat] <= (0.5 * ulp * scale)[~sat])
    np.testing.assert_array_equal(np.abs(dq[sat]), 448.0 * scale[sat])
    # dequantised weights are exactly representable in bf16 at these scales
    back = torch.from_numpy(dq).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(back, dq)
