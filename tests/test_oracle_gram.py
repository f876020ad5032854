"""Pins of the Gram form of the candidate loss ("AWQ：为什么 4-bit 权重量化要先观察 Activation",
§1: the exact layer-output squared error contains the cross terms of X^T X, which the
per-channel statistic a_j = mean |x_j| does not see).  The pins: the section's point as a
closed-form example (two inputs with the same statistic and errors 0 and 2), the identity
with the direct form sum (X E^T)^2 that the search oracle evaluates, and the algebra of G."""
import numpy as np
import pytest

from oracle import awq_oracle as o


def test_same_statistic_different_cross_terms():
    """Two one-token inputs with the same |x| per channel and one weight error e = (1, -1):
    the first cancels (output error 0), the second adds up (output error 2, squared 4).  The
    statistic cannot tell them apart; the Gram form gives both exactly."""
    e = np.array([[1.0, -1.0]])
    x1, x2 = np.array([[1.0, 1.0]]), np.array([[1.0, -1.0]])
    assert np.array_equal(o.activation_stat(x1), o.activation_stat(x2))
    assert o.gram_loss(o.gram_matrix(x1), 1, e) == 0.0
    assert o.gram_loss(o.gram_matrix(x2), 1, e) == 4.0
    # G of the second input by hand: [[1, -1], [-1, 1]]
    assert np.array_equal(o.gram_matrix(x2), np.array([[1.0, -1.0], [-1.0, 1.0]]))


def test_gram_matrix_is_the_sum_of_token_outer_products():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((7, 5))
    G = sum(np.outer(x, x) for x in X)
    assert np.allclose(o.gram_matrix(X), G, rtol=0, atol=1e-12)
    assert np.array_equal(o.gram_matrix(X), o.gram_matrix(X).T)
    assert np.all(np.linalg.eigvalsh(o.gram_matrix(X)) > -1e-12)  # positive semidefinite
    # token order does not matter
    assert np.allclose(o.gram_matrix(X[::-1]), o.gram_matrix(X), rtol=0, atol=1e-12)


@pytest.mark.parametrize("M,K,N,seed", [(64, 256, 128, 1), (300, 384, 40, 2), (5, 128, 3, 3)])
def test_gram_losses_equal_the_direct_losses(M, K, N, seed):
    rng = np.random.default_rng(seed)
    c = np.exp(0.5 * rng.standard_normal(K))
    X = rng.standard_normal((M, K)) * c
    W = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    a32 = o.activation_stat(X).astype(np.float32)
    ref = o.search(X, W, a32)
    g = o.gram_search_losses(X, W, ref["s_table"])
    assert np.allclose(g, ref["losses"], rtol=1e-10, atol=0)
    assert o.first_argmin(list(g)) == ref["best"] or \
        abs(ref["losses"][o.first_argmin(list(g))] - ref["losses"][ref["best"]]) <= 1e-10 * ref["losses"][ref["best"]]


def test_gram_loss_scales_with_the_square_of_x():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((20, 128))
    E = rng.standard_normal((6, 128))
    base = o.gram_loss(o.gram_matrix(X), 20, E)
    assert np.isclose(o.gram_loss(o.gram_matrix(3.0 * X), 20, E), 9.0 * base, rtol=1e-12)
    # and it equals the direct mean of (X E^T)^2
    assert np.isclose(base, np.mean((X @ E.T) ** 2), rtol=1e-12)
