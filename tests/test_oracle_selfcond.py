"""Pins for the self-conditioning oracle: one-hot, uniform and two-hot weights,
linearity, an element-by-element exact sum (math.fsum) on tiny inputs, and the
softmax mode against scipy's softmax.

Pages: [P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion LLM",
section "안정성을 위한 셀프 컨디셔닝"; [P3] section "Mehanizam odlučivanja o gotovim tokenima".
"""
import math

import numpy as np
import scipy.special

from oracle.selfcond import selfcond_embed, softmax_rows


def _e(V, d, seed=0):
    return (np.random.default_rng(seed).standard_normal((V, d)) * 0.02).astype(np.float32)


def test_one_hot_returns_the_row_exactly():
    """P-C1: a one-hot probability row returns exactly that embedding row."""
    E = _e(64, 16)
    p = np.zeros((3, 64))
    p[0, 5] = p[1, 0] = p[2, 63] = 1.0
    out = selfcond_embed(E, probs=p)
    for r, v in enumerate((5, 0, 63)):
        assert np.array_equal(out[r], E[v].astype(np.float64))


def test_uniform_returns_column_mean():
    """P-C2: p = 1/V returns the column mean of E."""
    E = _e(128, 8, 1)
    out = selfcond_embed(E, probs=np.full((1, 128), 1.0 / 128))
    np.testing.assert_allclose(out[0], E.astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-15)


def test_two_hot_and_linearity():
    """P-C4: weights 0.5/0.5 on a and b give (E[a] + E[b]) / 2; the map is linear."""
    E = _e(50, 12, 2)
    p = np.zeros((1, 50))
    p[0, 3] = p[0, 40] = 0.5
    out = selfcond_embed(E, probs=p)
    np.testing.assert_allclose(out[0], (E[3].astype(np.float64) + E[40]) / 2, rtol=1e-15)
    rng = np.random.default_rng(4)
    p1, p2 = rng.random((2, 50)), rng.random((2, 50))
    np.testing.assert_allclose(selfcond_embed(E, probs=2 * p1 - 3 * p2),
                               2 * selfcond_embed(E, probs=p1) - 3 * selfcond_embed(E, probs=p2), atol=1e-14)


def test_random_probs_against_exact_elementwise_sum():
    """P-C3: every output element equals the correctly rounded sum sum_v p[i,v] E[v,j]."""
    E = _e(40, 6, 3)
    rng = np.random.default_rng(5)
    p = rng.random((4, 40))
    p /= p.sum(axis=1, keepdims=True)
    out = selfcond_embed(E, probs=p)
    for i in range(4):
        for j in range(6):
            exact = math.fsum(float(p[i, v]) * float(E[v, j]) for v in range(40))
            assert abs(out[i, j] - exact) < 1e-15


def test_softmax_mode_equals_probability_mode():
    """P-C5: the logits mode is the probability mode on softmax(l); softmax itself is
    checked against scipy."""
    E = _e(256, 4, 6)
    rng = np.random.default_rng(7)
    l = rng.standard_normal((5, 256)) * np.array([0.1, 1, 3, 10, 30])[:, None]
    np.testing.assert_allclose(softmax_rows(l), scipy.special.softmax(l, axis=1), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(selfcond_embed(E, logits=l), selfcond_embed(E, probs=scipy.special.softmax(l, axis=1)),
                               rtol=1e-12, atol=1e-16)


def test_softmax_rows_are_independent():
    """Each row is normalised by its own maximum: rows 800 nats apart stay finite."""
    l = np.array([[800.0, 799.0, 798.0], [0.0, -1.0, -2.0]])
    p = softmax_rows(l)
    assert np.all(np.isfinite(p))
    np.testing.assert_allclose(p[0], p[1], rtol=1e-15)
