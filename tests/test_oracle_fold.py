"""Pins of the scale-folding oracle ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §6): the
page's GELU example (tests/golden/explainer_fold_example.json), the LayerNorm / Linear fold
algebra (exact with power-of-two scales), the odd-part identities of the activations and a
bit-level brute force of the bf16 rounding."""
import json
import os

import numpy as np
import pytest

from oracle import awq_oracle as o
from tests.conftest import GOLDEN

EX = json.load(open(os.path.join(GOLDEN, "explainer_fold_example.json")))


def test_gelu_example_matches_page():
    h = np.array([EX["h"]])
    s = np.array(EX["scales"], np.float32)
    Wkn = np.array(EX["weights_k_by_n"])
    W = Wkn.T  # [N, K]
    ref = o.gelu(h) @ W.T
    Ws = np.asarray(W, np.float64) * s[None, :].astype(np.float64)  # rows of the K x N weight times s
    correct = o.scaled_activation(h, s, "gelu") @ Ws.T
    wrong = o.gelu(h / s.astype(np.float64)[None, :]) @ Ws.T
    assert np.max(np.abs(correct - ref)) <= EX["correct_abs_tol"]
    assert np.max(np.abs(wrong - ref)) > EX["wrong_min_max_abs_diff"]


def test_layernorm_fold_is_exact_for_powers_of_two():
    rng = np.random.default_rng(0)
    K, N, M = 64, 16, 8
    Z = rng.standard_normal((M, K)).astype(np.float32)
    gamma = rng.standard_normal(K).astype(np.float32)
    beta = rng.standard_normal(K).astype(np.float32)
    W = rng.standard_normal((N, K)).astype(np.float32)
    s = np.exp2(rng.integers(-3, 4, K)).astype(np.float32)
    g2, b2 = o.fold_rows(gamma, s), o.fold_rows(beta, s)
    W2 = o.scale_cols(W, s)
    X = Z.astype(np.float64) * gamma + beta
    X2 = Z.astype(np.float64) * g2.astype(np.float64) + b2.astype(np.float64)
    assert np.array_equal(X2 @ W2.astype(np.float64).T, X @ W.astype(np.float64).T)
    # forgetting beta (the page's warning) changes the output
    X3 = Z.astype(np.float64) * g2.astype(np.float64) + beta
    assert np.max(np.abs(X3 @ W2.astype(np.float64).T - X @ W.astype(np.float64).T)) > 1e-3


def test_previous_linear_fold():
    rng = np.random.default_rng(1)
    K, Kin, N = 32, 48, 8
    Wp = rng.standard_normal((K, Kin)).astype(np.float32)
    bp = rng.standard_normal(K).astype(np.float32)
    W = rng.standard_normal((N, K)).astype(np.float32)
    s = np.exp2(rng.integers(-2, 3, K)).astype(np.float32)
    x = rng.standard_normal((4, Kin))
    ref = (x @ Wp.T.astype(np.float64) + bp) @ W.T.astype(np.float64)
    got = (x @ o.fold_rows(Wp, s).T.astype(np.float64) + o.fold_rows(bp, s)) @ o.scale_cols(W, s).T.astype(np.float64)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_fold_rounds_once():
    # a value whose quotient is not representable: one rounding of the exact quotient
    a = np.array([1.0, 2.0, 10.0], np.float32)
    s = np.array([3.0, 7.0, 3.0], np.float32)
    assert np.array_equal(o.fold_rows(a, s), np.array([1 / 3, 2 / 7, 10 / 3], np.float32))
    with pytest.raises(ValueError):
        o.fold_rows(a, np.array([1.0, 0.0, 2.0], np.float32))


def _bf16_brute(x: float) -> float:
    """Nearest bf16 by search over the neighbouring bf16 bit patterns (ties to even pattern)."""
    b = np.array([x], np.float32).view(np.uint32)[0] >> 16
    cands = [int(b) - 1, int(b), int(b) + 1, int(b) + 2]
    best = None
    for c in cands:
        v = float(np.array([c << 16], np.uint32).view(np.float32)[0])
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c, v)
    return best[2]


def test_bf16_rounding_brute_force():
    rng = np.random.default_rng(2)
    xs = np.concatenate([rng.standard_normal(500) * 10.0 ** rng.integers(-6, 6, 500),
                         [1.00390625, 1.005859375, -2.0078125, 0.3333333333333333]])
    got = o._round_to(xs, "bf16")
    for x, g in zip(xs, got):
        assert g == _bf16_brute(float(x)), x


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_activation_odd_part(act):
    f = {"gelu": o.gelu, "silu": o.silu}[act]
    x = np.linspace(-6, 6, 41)
    assert np.allclose(f(x) - f(-x), x, rtol=0, atol=1e-14)
    assert f(np.array([0.0]))[0] == 0.0


# Value pins for the two activations, fixed by mathematics rather than by the oracle's formula.
# The standard normal CDF gives Phi(1.6448536269514722) = 0.95 (the 95% quantile) and
# Phi(1) = 0.8413447460685429, and GELU(x) = x Phi(x).  The logistic function gives
# sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4, and SiLU(x) = x sigmoid(x).  A dropped sqrt(2)
# in the erfc argument, or a sign flip in the SiLU exponent, fails these.
@pytest.mark.parametrize("x,phi", [(1.6448536269514722, 0.95), (1.0, 0.8413447460685429),
                                   (-1.0, 1.0 - 0.8413447460685429), (-1.6448536269514722, 0.05)])
def test_gelu_normal_cdf_values(x, phi):
    got = float(o.gelu(np.array([x]))[0])
    assert got == pytest.approx(x * phi, rel=1e-14, abs=0)


def test_gelu_matches_library_normal_cdf():
    """GELU(x) = x Phi(x) against scipy's own normal CDF (scipy.special.ndtr) on [-10, 10]."""
    ndtr = pytest.importorskip("scipy.special").ndtr
    x = np.linspace(-10.0, 10.0, 2001)
    want = x * ndtr(x)
    got = o.gelu(x)
    nz = want != 0
    assert np.all(np.abs(got[nz] - want[nz]) <= 1e-13 * np.abs(want[nz]))


def test_silu_logistic_values():
    ln3 = np.log(3.0)
    got = o.silu(np.array([ln3, -ln3]))
    assert got[0] == pytest.approx(0.75 * ln3, rel=1e-15, abs=0)
    assert got[1] == pytest.approx(-0.25 * ln3, rel=1e-15, abs=0)


def test_silu_matches_library_logistic():
    """SiLU(x) = x sigmoid(x) against scipy's logistic function (scipy.special.expit)."""
    expit = pytest.importorskip("scipy.special").expit
    x = np.linspace(-30.0, 30.0, 1201)
    want = x * expit(x)
    got = o.silu(x)
    nz = want != 0
    assert np.all(np.abs(got[nz] - want[nz]) <= 1e-14 * np.abs(want[nz]))
