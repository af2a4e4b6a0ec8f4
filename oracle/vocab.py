"""Float64 CPU oracle for the steps on either side of the looped stack: the token
embedding, the LM head with its logit scale, and top-p sampling.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module. It shares no code with the HIP library and
imports neither it nor torch: inputs are NumPy arrays, arithmetic is float64.

What it computes ("Dory1.0-4B: A Looped Normalized-GPT"; page names as in the main
oracle module):

* embedding: the input state of token t is N(E_in[t]), the table row projected onto
  the unit sphere. nGPT keeps embeddings on the sphere (paper summary, "prerequisites:
  nGPT"), and the stack takes unit-norm states as its input.
* LM head: logits[v] = s_z[v] * (s . E_out[v]) for a final state s, with s_z the
  effective per-token logit scale (arXiv summary section 2 lists logit-scale parameters
  among the nGPT scales, initialised like the others). The effective vector is taken as
  given; how it is stored for training is out of scope.
* sampling: temperature T and nucleus (top-p) sampling with the generation settings of
  the MXFP8 article's deployment section (T = 1.0, top_p = 0.95): probabilities softmax(l / T);
  tokens ordered by probability, highest first, equal probabilities by lower id first;
  the nucleus is the shortest prefix of that order whose cumulative probability reaches
  top_p; one uniform draw u in [0, 1) per row selects the first nucleus token whose
  cumulative probability exceeds u times the nucleus mass (inverse CDF of the
  renormalised nucleus). The draws are inputs, so the result is a function of them.

The order of equal probabilities, "reaches" (>=) for the nucleus cut and "exceeds" (>)
for the draw are readings: the pages name the settings, not the procedure.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-12


def embed(table: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """N(table[id]) per id; ids outside [0, V) give a zero row (the boundary's rule for
    ids it cannot look up)."""
    table = np.asarray(table, dtype=np.float64)
    ids = np.asarray(ids).reshape(-1)
    out = np.zeros((ids.size, table.shape[1]))
    for i, t in enumerate(ids):
        if 0 <= t < table.shape[0]:
            row = table[t]
            out[i] = row / max(np.sqrt(np.sum(row * row)), EPS)
    return out


def logits(states: np.ndarray, lm_head: np.ndarray, logit_scale: np.ndarray) -> np.ndarray:
    """s_z[v] * (s . E_out[v]) for every state row s and token v."""
    s = np.asarray(states, dtype=np.float64)
    w = np.asarray(lm_head, dtype=np.float64)
    return (s @ w.T) * np.asarray(logit_scale, dtype=np.float64)[None, :]


def sorted_order(row: np.ndarray, temperature: float):
    """Token ids by probability (highest first, equal probabilities by lower id), the
    probabilities in that order and their running sum."""
    z = np.asarray(row, dtype=np.float64) / temperature
    e = np.exp(z - np.max(z))
    p = e / np.sum(e)
    ids = np.arange(p.size)
    order = np.lexsort((ids, -p))  # last key primary: -p ascending, then id ascending
    ps = p[order]
    return order, ps, np.cumsum(ps)


def nucleus_size(cum: np.ndarray, top_p: float) -> int:
    """Length of the shortest prefix whose cumulative probability reaches top_p (the
    whole vocabulary if rounding keeps the total below it)."""
    hit = np.nonzero(cum >= top_p)[0]
    return int(hit[0]) + 1 if hit.size else cum.size


def sample_top_p(row: np.ndarray, temperature: float, top_p: float, u: float) -> int:
    """The token the draw u selects from one row of logits."""
    order, _, cum = sorted_order(row, temperature)
    n = nucleus_size(cum, top_p)
    target = u * cum[n - 1]
    hit = np.nonzero(cum[:n] > target)[0]
    return int(order[hit[0]]) if hit.size else int(order[n - 1])


def sample_rows(lg: np.ndarray, temperature: float, top_p: float, u: np.ndarray) -> np.ndarray:
    return np.array([sample_top_p(lg[i], temperature, top_p, float(u[i])) for i in range(lg.shape[0])],
                    dtype=np.int64)


def draw_interval(row: np.ndarray, temperature: float, top_p: float, token: int):
    """For checking a sampler that sums in another precision: the position of `token`
    in the sorted order, the nucleus size, and the range [lo, hi) of u that selects it
    (lo = hi = nan when the token lies outside the nucleus)."""
    order, _, cum = sorted_order(row, temperature)
    n = nucleus_size(cum, top_p)
    rank = int(np.nonzero(order == token)[0][0])
    if rank >= n:
        return rank, n, float("nan"), float("nan")
    mass = cum[n - 1]
    lo = (cum[rank - 1] if rank else 0.0) / mass
    return rank, n, lo, cum[rank] / mass
