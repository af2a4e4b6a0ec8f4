"""NVFP4 weight format (W4A16), CPU oracle. TEST INFRASTRUCTURE ONLY.

The pages give NVFP4 as NVIDIA's 4-bit block-scaled format, E2M1 elements with E4M3
scale factors (paper summary, "NVFP4 quantisation and QAD"), used weight-only (W4A16,
model-card digest, quantised versions) and quantised with dynamic MSE scale selection
while the other formats use maximum scaling (arXiv summary 5.1-5.2). Embeddings, LM head,
vectors and scalars stay in high precision.

Readings for what the pages leave open:
* E2M1: sign, 2 exponent bits, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
  no infinities or NaN. Elements round to the nearest magnitude, ties to the even code,
  beyond 6 saturate to 6; the sign bit is kept.
* blocks of 16 consecutive elements along the input (K) axis of each [N_out, K_in]
  matrix, one E4M3 scale byte each (the OCP "FN" E4M3 of the MXFP8 oracle).
* a per-matrix scale g on top of the block scales, so that small weights do not fall into
  E4M3's subnormal range: g = 2^ceil(log2(amax / (6 * 448))), a power of two, so that the
  block scale amax/6/g a maximum-scaled block would need is at most 448. Being a power
  of two, g keeps every dequantised weight e2m1 * e4m3 * g exactly representable in
  bfloat16 (and float32); g = 1 for an all-zero matrix.
* "MSE scale selection": each block takes, among all positive finite E4M3 scale codes
  (0x01..0x7E), the one whose dequantised block has the smallest sum of squared errors;
  equal sums go to the smaller code. The decision is an integer chosen by floating-point
  comparisons, so it is taken in float32 with a fixed order, as the GPU takes it: for
  each element x = w / S (S = e4m3 * g, exact), q = E2M1(x), d = q * S - w, and the sum
  adds d * d element by element (each product and sum rounded, no fused multiply-add).
* packing: byte j of a row holds elements 2j (low nibble) and 2j + 1 (high nibble).
"""
from __future__ import annotations

import numpy as np

from .mxfp8 import e4m3_decode

BLOCK = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
SCALE_CODES = np.arange(1, 0x7F, dtype=np.int64)  # positive finite E4M3 codes


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    return np.where(c & 8, -1.0, 1.0) * E2M1_VALUES[c & 7]


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code of each value (ties to the even code, saturation at 6, sign
    kept). Comparisons against midpoints, which are exact in any binary format."""
    x = np.asarray(x)
    a = np.abs(x.astype(np.float64))
    # midpoints between consecutive magnitudes; at a tie the even code (lower index
    # 0, 2, 4, 6 or upper index 2, 4, 6) wins
    mids = (E2M1_VALUES[:-1] + E2M1_VALUES[1:]) / 2   # 0.25 0.75 1.25 1.75 2.5 3.5 5
    mag = np.zeros(a.shape, dtype=np.int64)
    for i, m in enumerate(mids):
        lower_even = i % 2 == 0       # codes i (lower) and i + 1 (upper)
        mag = np.where((a > m) | ((a == m) & (not lower_even)), i + 1, mag)
    return np.where(np.signbit(x), 8, 0) + mag


def global_scale(w: np.ndarray) -> np.float32:
    """g = 2^ceil(log2(amax / 2688)) in float32 (1 for an all-zero matrix)."""
    amax = np.float32(np.max(np.abs(np.asarray(w, dtype=np.float32)))) if np.size(w) else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    r = np.float32(amax / np.float32(E2M1_MAX * E4M3_MAX))
    f, e = np.frexp(r)              # r = f 2^e, f in [0.5, 1)
    return np.float32(np.ldexp(1.0, int(e) - 1 if f == 0.5 else int(e)))


def quantize(w: np.ndarray):
    """NVFP4 codes of a [N, K] matrix (K % 16 == 0): packed E2M1 codes [N, K/2] (uint8),
    E4M3 block scales [N, K/16] (uint8) and the per-matrix scale g (float32)."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % BLOCK == 0
    g = global_scale(w)
    blocks = w.reshape(N, K // BLOCK, BLOCK)
    best_err = np.full(blocks.shape[:2], np.inf, dtype=np.float32)
    best_code = np.zeros(blocks.shape[:2], dtype=np.int64)
    for c in SCALE_CODES:
        S = np.float32(np.float32(e4m3_decode(c)) * g)  # exact: E4M3 value times a power of two
        err = np.zeros(blocks.shape[:2], dtype=np.float32)
        for i in range(BLOCK):
            wi = blocks[:, :, i]
            x = wi / S                                   # float32 IEEE division
            q = e2m1_decode(e2m1_encode(x)).astype(np.float32)
            d = q * S - wi                               # q * S exact; one rounding in the difference
            err = err + d * d                            # product and sum each rounded
        better = err < best_err                          # strict: equal sums keep the smaller code
        best_err = np.where(better, err, best_err)
        best_code = np.where(better, c, best_code)
    S = (e4m3_decode(best_code).astype(np.float32) * g).astype(np.float32)
    q = e2m1_encode(blocks / S[:, :, None]).reshape(N, K)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, best_code.astype(np.uint8), g


def unpack(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.int64)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int64)
    out[:, 0::2] = p & 15
    out[:, 1::2] = p >> 4
    return out


def dequantize(packed: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    """W = e2m1 * e4m3 * g (float64, exact)."""
    q = e2m1_decode(unpack(packed))
    s = np.repeat(e4m3_decode(np.asarray(scales, dtype=np.int64)), BLOCK, axis=1)
    return q * s * float(g)


def block_errors_f64(w_block: np.ndarray, g: float) -> np.ndarray:
    """Sum of squared errors (float64) of one block for every candidate scale code, each
    element taking its nearest E2M1 value (for the tests)."""
    w = np.asarray(w_block, dtype=np.float64)
    grid = np.concatenate([-E2M1_VALUES[::-1], E2M1_VALUES])
    out = []
    for c in SCALE_CODES:
        S = float(e4m3_decode(c)) * g
        near = np.min(np.abs(grid[None, :] * S - w[:, None]), axis=1)  # nearest point of the scaled grid
        out.append(float(np.sum(near ** 2)))
    return np.array(out)
