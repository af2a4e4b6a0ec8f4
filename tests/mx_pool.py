"""The oracle's MXFP8 round trip of several weight matrices in worker processes.

The quantiser (oracle/mxfp8.py) handles about five million weights a second in
NumPy; the 72-layer parity cases quantise a few hundred million, so the matrices go
to a pool of fresh ("spawn") interpreters that import only NumPy and the oracle. The
workers never touch the GPU."""
from __future__ import annotations

import multiprocessing as mp
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def _round_trip(w32: np.ndarray) -> np.ndarray:
    from oracle import mxfp8 as MX
    codes, scales = MX.quantize(np.asarray(w32, dtype=np.float64))
    # dequantised MXFP8 values (3 mantissa bits times a power of two) are exact in float32
    return MX.dequantize(codes, scales).astype(np.float32)


def dequantised_many(mats: list, workers: int = 8) -> list:
    """dequantize(quantize(w)) for each float32 matrix, in order (float32 results)."""
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=min(workers, len(mats)), mp_context=ctx) as ex:
        return list(ex.map(_round_trip, mats))
