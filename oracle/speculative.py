"""Float64 CPU oracle for self-speculative decoding's acceptance step.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module. It shares no code with the HIP library and
imports neither it nor torch.

The pages ("Dory1.0-4B: A Looped Normalized-GPT"; arXiv summary 6.2, paper summary
experiments) draft gamma = 4 tokens with one loop and verify them with k loops, and
keep the k-loop output distribution by rejection sampling. Written here as standard
speculative sampling over the distributions the generation settings give (temperature,
then the top-p nucleus renormalised; the vocabulary oracle's definitions):

* draft token j (j = 1..gamma) was drawn from q_j, the draft model's processed
  distribution at that position; p_j is the verifying model's at the same position.
* it is accepted when u_j < p_j(x_j) / q_j(x_j) (always when p_j(x_j) >= q_j(x_j));
  at the first rejection the step emits one token drawn from the residual
  max(0, p_j - q_j), renormalised, and stops;
* if all gamma are accepted, one more token is drawn from p_{gamma+1}.
* draws: the residual by inverse CDF over token ids in increasing order (the first id
  whose running residual mass exceeds u times the total); the extra token with the
  vocabulary oracle's top-p sampler. The order of the inverse CDF is a reading; any fixed
  order samples the same distribution.

Each emitted token is then distributed as p at its position: the draft only changes how
many tokens one verification yields.
"""
from __future__ import annotations

import numpy as np

from . import vocab as V


def processed(row: np.ndarray, temperature: float, top_p: float) -> np.ndarray:
    """The distribution a row of logits gives after temperature and top-p: nucleus
    probabilities renormalised, zero elsewhere (float64, by token id)."""
    order, ps, cum = V.sorted_order(row, temperature)
    n = V.nucleus_size(cum, top_p)
    out = np.zeros(ps.size)
    out[order[:n]] = ps[:n] / cum[n - 1]
    return out


def residual_draw(p: np.ndarray, q: np.ndarray, u: float) -> int:
    """The token u draws from max(0, p - q) renormalised (inverse CDF by increasing id;
    if the residual is empty, which needs p == q, from p itself)."""
    r = np.maximum(p - q, 0.0)
    if r.sum() <= 0.0:
        r = p.copy()
    cum = np.cumsum(r)
    hit = np.nonzero(cum > u * cum[-1])[0]
    return int(hit[0]) if hit.size else int(np.nonzero(r > 0)[0][-1])


def accept(draft_logits: np.ndarray, target_logits: np.ndarray, draft_tokens, temperature: float,
           top_p: float, u_accept, u_sample: float):
    """One sequence: draft_logits [gamma, V] (the rows the draft tokens were drawn from),
    target_logits [gamma + 1, V] (the verifying model at the same positions and one
    more), draft_tokens [gamma]. Returns (number accepted, emitted tokens: the accepted
    drafts then one more)."""
    gamma = len(draft_tokens)
    out = []
    for j in range(gamma):
        x = int(draft_tokens[j])
        p = processed(target_logits[j], temperature, top_p)
        q = processed(draft_logits[j], temperature, top_p)
        ratio = p[x] / q[x] if q[x] > 0 else 0.0
        if u_accept[j] < ratio:
            out.append(x)
            continue
        out.append(residual_draw(p, q, float(u_sample)))
        return j, out
    out.append(V.sample_top_p(target_logits[gamma], temperature, top_p, float(u_sample)))
    return gamma, out
