"""Pins for the oracle's primitives: closed forms, special cases and independent
library routines (not the ones the oracle calls)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import dory_oracle as O
from tests.helpers import TINY

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


def facts():
    with open(GOLDEN) as f:
        return json.load(f)


def test_l2n_closed_form():
    np.testing.assert_allclose(O.l2n(np.array([[3.0, 4.0]])), [[0.6, 0.8]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(O.l2n(np.array([[0.0, -2.0, 0.0]])), [[0.0, -1.0, 0.0]], atol=0)
    z = O.l2n(np.zeros((2, 5)))                      # N(0) reading: zero stays zero
    assert np.all(z == 0)
    r = np.random.default_rng(0).standard_normal((7, 33)) * 1e3
    np.testing.assert_allclose(np.linalg.norm(O.l2n(r), axis=1), 1.0, atol=1e-14)


def test_nonlinearities_against_scipy():
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.sigmoid(z), scipy.special.expit(z), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-13, atol=1e-300)
    assert O.silu(np.array(0.0)) == 0.0
    assert O.sigmoid(np.array(0.0)) == 0.5
    a = np.random.default_rng(1).standard_normal((5, 17)) * 20
    np.testing.assert_allclose(O.softmax(a), scipy.special.softmax(a, axis=-1), rtol=1e-13)


def test_ngpt_update_special_cases():
    rng = np.random.default_rng(2)
    s = O.l2n(rng.standard_normal((4, 12)))
    h = rng.standard_normal((4, 12)) * 3.0
    np.testing.assert_allclose(O.ngpt_update(s, h, np.zeros(12)), s, atol=1e-15)     # a=0: keep
    np.testing.assert_allclose(O.ngpt_update(s, h, np.ones(12)), O.l2n(h), atol=1e-15)  # a=1: N(h)
    # two-channel worked case: s=e1, h=2*e2, a=1/2 -> N(e1/2 + e2/2) = (1,1)/sqrt2
    out = O.ngpt_update(np.array([[1.0, 0.0]]), np.array([[0.0, 2.0]]), np.array([0.5, 0.5]))
    np.testing.assert_allclose(out, [[2 ** -0.5, 2 ** -0.5]], atol=1e-15)
    # per-channel rates act per channel: a=(1,0) with s=e1 and h=e2 -> (1-1)*1, (1-0)*0 + ...
    out = O.ngpt_update(np.array([[0.6, 0.8]]), np.array([[0.0, 5.0]]), np.array([1.0, 0.0]))
    np.testing.assert_allclose(out, [[0.0, 1.0]], atol=1e-15)


def test_rope_against_complex_rotation():
    """Half-split pairs (i, i+d/2) rotated by p * theta^(-2i/d) equal multiplying the
    complex number x_i + j x_{i+d/2} by exp(j p theta^(-2i/d))."""
    rng = np.random.default_rng(3)
    T, Hh, d = 6, 3, 16
    x = rng.standard_normal((T, Hh, d))
    pos = np.array([0, 1, 7, 100, 4096, 131071])
    theta = 1e4
    out = O.rope(x, pos, theta)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    f = np.array([theta ** (-2.0 * i / d) for i in range(d // 2)])
    zr = z * np.exp(1j * pos[:, None, None] * f[None, None, :])
    np.testing.assert_allclose(out[..., : d // 2], zr.real, atol=1e-12)
    np.testing.assert_allclose(out[..., d // 2:], zr.imag, atol=1e-12)


def test_rope_properties():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 2, 8))
    np.testing.assert_allclose(O.rope(x, np.zeros(5, int), 1e7), x, atol=0)        # p=0: identity
    y = O.rope(x, np.arange(5) * 37, 1e4)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    # d=2: a single pair with frequency 1 -> (cos p, sin p)
    np.testing.assert_allclose(O.rope(np.array([[[1.0, 0.0]]]), np.array([1]), 1e4),
                               [[[math.cos(1.0), math.sin(1.0)]]], atol=1e-15)
    # logits depend on p - j only
    q, k = rng.standard_normal((1, 1, 8)), rng.standard_normal((1, 1, 8))
    d1 = np.sum(O.rope(q, np.array([50]), 1e4) * O.rope(k, np.array([20]), 1e4))
    d2 = np.sum(O.rope(q, np.array([1030]), 1e4) * O.rope(k, np.array([1000]), 1e4))
    assert abs(d1 - d2) < 1e-12


def test_pages_structural_facts():
    F = facts()
    c72 = O.Config.from_dict(dict(TINY, n_in=16, n_rec=40, n_out=16))
    for k, e in F["effective_depth_72"]["value"].items():
        assert O.effective_depth(c72, int(k)) == e
    assert [c72.n_in, c72.n_rec, c72.n_out] == F["block_split_72"]["value"]
    assert c72.n_layers == 72
    c36 = O.Config.from_dict(dict(TINY, n_in=8, n_rec=20, n_out=8))
    full = sum(O.layer_is_full(c36, i) for i in range(36))
    assert {"sliding": 36 - full, "full": full} == F["attention_layers_36"]["value"]
    # the pattern: three sliding then one full, from the first layer on
    assert [O.layer_is_full(c36, i) for i in range(8)] == [False, False, False, True] * 2
    # last_loop slots do not depend on k; per_loop slots grow with k
    assert F["last_loop_kv_one_loop_size"]["value"]
    assert len({O.attn_slots(c72, k, "last_loop") for k in (1, 2, 4)}) == 1
    assert O.attn_slots(c72, 1, "last_loop") == O.attn_slots(c72, 1, "per_loop") == 72
    assert O.attn_slots(c72, 4, "per_loop") == 16 + 16 + 4 * 40
