"""Pins for the vocabulary oracle (embedding, LM head, top-p sampling): hand-worked
cases of the definition, textbook limits (greedy, plain inverse-CDF sampling), an
independent brute-force dot product, and invariances."""
import math

import numpy as np
import pytest
import scipy.special

from oracle import vocab as V


def test_embed_unit_rows_and_invalid_ids():
    table = np.array([[3.0, 4.0, 0.0], [0.0, 0.0, -2.0], [1.0, 1.0, 1.0]])
    out = V.embed(table, np.array([0, 2, -1, 3, 1]))
    np.testing.assert_allclose(out[0], [0.6, 0.8, 0.0], atol=1e-15)
    np.testing.assert_allclose(out[1], np.full(3, 1 / math.sqrt(3)), atol=1e-15)
    assert np.all(out[2] == 0) and np.all(out[3] == 0)     # ids outside [0, V)
    np.testing.assert_allclose(out[4], [0.0, 0.0, -1.0], atol=0)
    r = np.random.default_rng(3).standard_normal((50, 40)) * 7
    np.testing.assert_allclose(np.linalg.norm(V.embed(r, np.arange(50)), axis=1), 1.0, atol=1e-14)


def test_logits_against_brute_force_loops():
    rng = np.random.default_rng(4)
    s, w, z = rng.standard_normal((3, 5)), rng.standard_normal((4, 5)), rng.uniform(0.5, 2, 4)
    got = V.logits(s, w, z)
    for i in range(3):
        for v in range(4):
            acc = 0.0
            for c in range(5):
                acc += s[i, c] * w[v, c]
            assert abs(got[i, v] - z[v] * acc) < 1e-13


def test_worked_example():
    # p = (0.5, 0.3, 0.2); with top_p 0.75 the nucleus is {0, 1} (0.5 + 0.3 reaches it),
    # mass 0.8; u selects by u * 0.8 against the running sums 0.5, 0.8
    lg = np.log(np.array([0.5, 0.3, 0.2]))
    assert V.sample_top_p(lg, 1.0, 0.75, 0.0) == 0
    assert V.sample_top_p(lg, 1.0, 0.75, 0.6) == 0       # 0.48 < 0.5
    assert V.sample_top_p(lg, 1.0, 0.75, 0.7) == 1       # 0.56
    assert V.sample_top_p(lg, 1.0, 0.75, 0.999) == 1     # token 2 is outside the nucleus
    # the cut "reaches": top_p equal to a running sum ends the nucleus there
    assert V.sample_top_p(lg, 1.0, 0.8 - 1e-12, 0.999) == 1
    assert V.sample_top_p(lg, 1.0, 0.81, 0.999) == 2
    # order is by probability, not by id
    lg2 = np.log(np.array([0.2, 0.5, 0.3]))
    assert V.sample_top_p(lg2, 1.0, 0.75, 0.0) == 1
    assert V.sample_top_p(lg2, 1.0, 0.75, 0.7) == 2
    rank, n, lo, hi = V.draw_interval(lg2, 1.0, 0.75, 2)
    assert (rank, n) == (1, 2) and abs(lo - 0.625) < 1e-12 and abs(hi - 1.0) < 1e-12
    assert math.isnan(V.draw_interval(lg2, 1.0, 0.75, 0)[2])


def test_equal_probabilities_go_by_id():
    lg = np.zeros(10)
    # nucleus of 10 equal tokens at top_p 0.35 is the first 4 ids (0.3 < 0.35 <= 0.4)
    got = [V.sample_top_p(lg, 1.0, 0.35, u) for u in (0.0, 0.24, 0.26, 0.74, 0.76, 0.99)]
    assert got == [0, 0, 1, 2, 3, 3]


def test_tiny_top_p_is_greedy():
    rng = np.random.default_rng(5)
    for _ in range(20):
        lg = rng.standard_normal(300) * 3
        for u in (0.0, 0.5, 0.999):
            assert V.sample_top_p(lg, 1.0, 1e-9, u) == int(np.argmax(lg))


def test_full_nucleus_is_plain_inverse_cdf():
    # top_p = 1: over a fine grid of draws each token is chosen in proportion to its
    # softmax probability (computed independently with scipy)
    rng = np.random.default_rng(6)
    lg = rng.standard_normal(40) * 2
    p = scipy.special.softmax(lg)
    n = 20000
    counts = np.bincount([V.sample_top_p(lg, 1.0, 1.0, (i + 0.5) / n) for i in range(n)], minlength=40)
    assert np.all(np.abs(counts - n * p) <= 1.0 + 1e-9)


def test_nucleus_distribution_on_a_grid():
    # top_p = 0.9: the draws reproduce the renormalised nucleus of the sorted order
    rng = np.random.default_rng(7)
    lg = rng.standard_normal(60) * 1.5
    p = scipy.special.softmax(lg)
    idx = sorted(range(60), key=lambda i: (-p[i], i))
    c, keep = 0.0, []
    for i in idx:
        keep.append(i)
        c += p[i]
        if c >= 0.9:
            break
    q = np.zeros(60)
    q[keep] = p[keep] / p[keep].sum()
    n = 20000
    counts = np.bincount([V.sample_top_p(lg, 1.0, 0.9, (i + 0.5) / n) for i in range(n)], minlength=60)
    assert np.all(np.abs(counts - n * q) <= 1.0 + 1e-9)


def test_temperature_divides_logits():
    rng = np.random.default_rng(8)
    lg = rng.standard_normal(200) * 4
    for u in np.linspace(0, 0.999, 23):
        assert V.sample_top_p(lg, 2.0, 0.95, u) == V.sample_top_p(lg / 2.0, 1.0, 0.95, u)
    # a high temperature flattens the distribution: the nucleus grows
    _, _, c1 = V.sorted_order(lg, 1.0)
    _, _, c5 = V.sorted_order(lg, 5.0)
    assert V.nucleus_size(c5, 0.95) > V.nucleus_size(c1, 0.95)


def test_relabelling_tokens_relabels_the_choice():
    rng = np.random.default_rng(9)
    lg = rng.standard_normal(500) * 3
    perm = rng.permutation(500)
    for u in np.linspace(0, 0.999, 31):
        a = V.sample_top_p(lg, 1.0, 0.95, u)
        b = V.sample_top_p(lg[perm], 1.0, 0.95, u)   # token j of the copy is token perm[j]
        assert perm[b] == a
