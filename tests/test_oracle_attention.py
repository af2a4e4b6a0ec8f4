"""Attention-sublayer pins for the oracle: brute force on tiny shapes, special cases
and invariances the method's definition fixes."""
import copy

import numpy as np
import pytest

from oracle import dory_oracle as O
from tests.bruteforce import BruteModel, weights_to_lists
from tests.helpers import SMALL, TINY, inputs, model


def _attn_only(cfg, lw, X, pos, layer, kv=None, slot=0):
    kv = kv if kv is not None else O.KVStore(cfg)
    return O.attention(cfg, lw, X, pos, layer, kv, slot)


@pytest.mark.parametrize("qk_norm,gate", [(1, 1), (0, 1), (1, 0), (0, 0)])
@pytest.mark.parametrize("layer", [0, 3])          # sliding (window 3) and full
def test_attention_matches_bruteforce(qk_norm, gate, layer):
    cd = dict(TINY, qk_norm=qk_norm, attn_gate=gate,
              attn_scale=(TINY["attn_scale"] if qk_norm else 8 ** -0.5))
    cfg, W, packed = model(cd, seed=11)
    X = inputs(cd, 7, seed=5)
    pos = np.arange(7)
    y = _attn_only(cfg, W[layer], X, pos, layer)
    bm = BruteModel(cd, weights_to_lists(cd, packed))
    yb = bm._attn(layer, 0, X.tolist(), list(range(7)))
    np.testing.assert_allclose(y, np.array(yb), rtol=0, atol=1e-13)


def test_sliding_equals_full_when_window_covers_sequence():
    cfg, W, _ = model(TINY, seed=12)
    X = inputs(TINY, 9, seed=6)
    pos = np.arange(9)
    wide = copy.copy(cfg)
    wide.window = 9
    full_like = copy.copy(cfg)
    full_like.full_period = 1          # every layer full
    full_like.theta_full = cfg.theta_swa
    a = _attn_only(wide, W[0], X, pos, 0)
    b = _attn_only(full_like, W[0], X, pos, 0)
    np.testing.assert_allclose(a, b, atol=1e-14)
    narrow = _attn_only(cfg, W[0], X, pos, 0)      # window 3 < 9 must differ
    assert np.abs(narrow - a).max() > 1e-6


def test_single_token_output_is_value():
    """T = 1: softmax over one key is 1, so the head outputs are that token's v."""
    cd = dict(TINY, attn_gate=0)
    cfg, W, _ = model(cd, seed=13)
    cfg.pre_proj_norm = False
    lw = copy.copy(W[0])
    lw.wo = np.eye(cfg.hidden)
    X = inputs(cd, 1, seed=7)
    y = _attn_only(cfg, lw, X, np.array([0]), 0)
    v = (X @ W[0].wv.T).reshape(1, cfg.n_kv_heads, cfg.head_dim)
    expect = np.repeat(v, cfg.n_q_heads // cfg.n_kv_heads, axis=1).reshape(1, -1)
    np.testing.assert_allclose(y, expect, atol=1e-15)


def test_gqa_equals_mha_with_repeated_kv_heads():
    cfg, W, _ = model(SMALL, seed=14)            # 4 query heads over 2 KV heads
    X = inputs(SMALL, 6, seed=8)
    pos = np.arange(6)
    mha = copy.copy(cfg)
    mha.n_kv_heads = cfg.n_q_heads
    lw = copy.copy(W[0])
    d = cfg.head_dim
    rep = lambda w: np.concatenate([w[(h // 2) * d:(h // 2 + 1) * d] for h in range(4)])
    lw.wk, lw.wv = rep(W[0].wk), rep(W[0].wv)
    np.testing.assert_allclose(_attn_only(cfg, W[0], X, pos, 0),
                               _attn_only(mha, lw, X, pos, 0), atol=1e-14)


def test_causality():
    cfg, W, _ = model(TINY, seed=15)
    X = inputs(TINY, 10, seed=9)
    full = _attn_only(cfg, W[3], X, np.arange(10), 3)
    part = _attn_only(cfg, W[3], X[:6], np.arange(6), 3)
    np.testing.assert_allclose(full[:6], part, atol=1e-15)


def test_unwritten_kv_read_raises():
    cfg, W, _ = model(TINY, seed=17)
    kv = O.KVStore(cfg)
    with pytest.raises(KeyError):
        kv.read(0, 0, 0, 3)
