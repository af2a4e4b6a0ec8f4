"""Pins for the speculative-acceptance oracle: identical draft and target accept every
draft token; tokens outside the target's nucleus are always rejected; the residual draw
on hand-worked cases; and the defining property, checked on a grid of draws: the first
emitted token is distributed as the target's processed distribution, whatever the
draft."""
import numpy as np

from oracle import speculative as SP
from oracle import vocab as V


def test_same_model_accepts_everything():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((5, 50)) * 2
    toks = [V.sample_top_p(lg[j], 1.0, 0.95, 0.3 + 0.1 * j) for j in range(4)]
    for ua in (0.0, 0.5, 0.999):
        a, out = SP.accept(lg[:4], lg, toks, 1.0, 0.95, [ua] * 4, 0.42)
        assert a == 4 and out[:4] == toks
        assert out[4] == V.sample_top_p(lg[4], 1.0, 0.95, 0.42)


def test_token_outside_target_nucleus_is_rejected():
    tgt = np.log(np.array([[0.6, 0.39, 0.01], [0.6, 0.39, 0.01]]))
    drf = np.log(np.array([[0.2, 0.2, 0.6]]))
    for ua in (0.0, 0.5):
        a, out = SP.accept(drf, tgt, [2], 1.0, 0.95, [ua], 0.1)   # token 2 is outside p's nucleus
        assert a == 0 and len(out) == 1 and out[0] in (0, 1)


def test_residual_draw_cases():
    p, q = np.array([0.5, 0.3, 0.2]), np.array([0.2, 0.5, 0.3])
    assert all(SP.residual_draw(p, q, u) == 0 for u in (0.0, 0.5, 0.99))      # residual [0.3, 0, 0]
    p, q = np.array([0.3, 0.5, 0.2]), np.array([0.1, 0.2, 0.7])                # residual [0.2, 0.3, 0]
    assert SP.residual_draw(p, q, 0.39) == 0 and SP.residual_draw(p, q, 0.41) == 1
    assert SP.residual_draw(p, p, 0.7) == 1                                    # empty residual: from p


def test_processed_distribution():
    lg = np.log(np.array([0.5, 0.3, 0.15, 0.05]))
    np.testing.assert_allclose(SP.processed(lg, 1.0, 0.75), [0.625, 0.375, 0, 0], atol=1e-15)
    np.testing.assert_allclose(SP.processed(lg, 1.0, 1.0), [0.5, 0.3, 0.15, 0.05], atol=1e-15)


def test_first_token_follows_the_target():
    # a draft far from the target; stratified grids over the draft's draw, the acceptance
    # draw and the residual draw: the first emitted token's frequencies are p's
    tgt = np.log(np.array([[0.45, 0.25, 0.2, 0.1], [0.25, 0.25, 0.25, 0.25]]))
    drf = np.log(np.array([[0.1, 0.2, 0.3, 0.4]]))
    p = SP.processed(tgt[0], 1.0, 1.0)
    n = 40
    grid = (np.arange(n) + 0.5) / n
    counts = np.zeros(4)
    for ud in grid:
        x = V.sample_top_p(drf[0], 1.0, 1.0, ud)
        for ua in grid:
            for us in grid:
                counts[SP.accept(drf, tgt, [x], 1.0, 1.0, [ua], us)[1][0]] += 1
    np.testing.assert_allclose(counts / n ** 3, p, atol=0.02)
