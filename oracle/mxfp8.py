"""MXFP8 weight format, float64 CPU oracle. TEST INFRASTRUCTURE ONLY.

The pages give the checkpoint's format as W8A16 MXFP8: E4M3 weight elements with
one shared scale per group of 32 ("group_size 32" in the MXFP8 article's config
list), quantised from BF16 with standard maximum scaling (arXiv summary 5.1-5.2),
applied to the weight matrices while vectors and scalars stay in high precision.

Reading for the parts the pages leave open (OCP Microscaling formats v1.0):
* E4M3 is the OCP "FN" variant: bias 7, subnormals m * 2^-9, max normal 448,
  code S.1111.111 is NaN, no infinities.
* shared scale X = 2^(floor(log2(amax)) - 8), 8 being E4M3's largest normal
  exponent, stored as the E8M0 byte floor(log2(amax)) - 8 + 127, clamped to
  [0, 254]; an all-zero group stores byte 0.
* elements are x / X rounded to the nearest E4M3 value, ties to the even code,
  magnitudes beyond 448 saturate to 448; the sign bit is kept (a negative value
  that rounds to zero encodes as 0x80).
* groups run along the input (K) axis of each [N_out, K_in] matrix.

The encoder rounds by looking up the two neighbouring values in the table of all
finite E4M3 values; the tests pin it against an exhaustive nearest-value search.
"""
from __future__ import annotations

import numpy as np

GROUP = 32
E4M3_MAX = 448.0
EMAX_ELEM = 8


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Value of each E4M3 byte (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


# all non-negative finite codes 0x00..0x7E and their values
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = e4m3_decode(_POS_CODES)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to even code, saturate at 448.

    The finite non-negative values increase strictly with the code, so the two
    candidates for |x| are the table neighbours found by binary search.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALS, a, side="left"), 0, len(_POS_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - a
    code = np.where(dhi < dlo, hi, lo)
    tie = (dhi == dlo) & (hi != lo)
    code = np.where(tie, np.where(hi % 2 == 0, hi, lo), code)   # ties: even mantissa
    code = np.where(a == _POS_VALS[hi], hi, code)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    return np.exp2(np.asarray(b, dtype=np.float64) - 127.0)


def quantize(w: np.ndarray):
    """Quantise a [N, K] matrix (K % 32 == 0). Returns (codes uint8 [N,K],
    scales uint8 [N, K/32])."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    assert K % GROUP == 0
    g = w.reshape(N, K // GROUP, GROUP)
    amax = np.abs(g).max(axis=-1)
    # floor(log2(amax)) exactly: amax = f * 2^e with f in [0.5, 1)
    _, e = np.frexp(amax)
    se = np.where(amax > 0, (e - 1).astype(np.float64) - EMAX_ELEM, -127.0)
    se = np.clip(se, -127, 127)
    scales = (se + 127).astype(np.uint8)
    codes = e4m3_encode(g / np.exp2(se)[..., None]).reshape(N, K)
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W = E4M3(code) * 2^(scale - 127), float64 [N, K]."""
    N, K = codes.shape
    v = e4m3_decode(codes).reshape(N, K // GROUP, GROUP)
    return (v * e8m0_decode(scales)[..., None]).reshape(N, K)
