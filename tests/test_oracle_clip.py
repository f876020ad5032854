"""Pins of the clipping-search oracle ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §5):
the page's per-group counterexample (tests/golden/explainer_clip_example.json), a vector
derived by hand in the fp32 contract, exact rational errors on tiny shapes, invariants and
the first-minimum rule."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import awq_oracle as o
from tests.conftest import GOLDEN

EX = json.load(open(os.path.join(GOLDEN, "explainer_clip_example.json")))


# ------------------------------------------------------------------ teaching counterexample
def test_teaching_counterexample_matches_page():
    groups = [(g["x"], g["w"]) for g in EX["groups"]]
    res = o.teaching_clip_search(groups, EX["n_candidates"])
    refs = [r for _, _, r in res]
    assert abs(sum(refs) - EX["whole_output"]) <= 1e-12
    base = [sum(a * b for a, b in zip(x, o.teaching_clip_qdq(w, 1.0))) for x, w in groups]
    assert abs(sum(base) - EX["baseline_sum"]) <= 1e-12  # the two baseline errors cancel
    sel = sum(p for _, p, _ in res)
    exact = EX["selected_sum_exact"]
    assert abs(sel - exact["num"] / exact["den"]) <= 1e-12
    assert round(sel, 9) == EX["selected_sum_printed"]
    d = EX["printed_decimals"]
    for (x, w), b, (f, p, r) in zip(groups, base, res):
        assert round(abs(b - r), d) == EX["group_abs_error_before_printed"]
        assert round(abs(p - r), d) == EX["group_abs_error_after_printed"]
        assert (p - r) ** 2 < (b - r) ** 2  # every group improves ...
        assert f < 1.0
    # ... while the whole output gets worse
    assert (sel - EX["whole_output"]) ** 2 > (sum(base) - EX["whole_output"]) ** 2


def test_teaching_factor_one_is_the_plain_teaching_quantizer():
    for vals in ([0.1, 0.2], [-1.0, 0.5, 0.25, 1.0], [3.0, -0.5, 0.0], [0.0, 0.0]):
        assert o.teaching_clip_qdq(vals, 1.0) == o.teaching_qdq(vals)[1]


@pytest.mark.parametrize("vals,f", [([float("nan"), 1.0], 1.0), ([1.0], 0.0), ([1.0], 1.5), ([], 1.0)])
def test_teaching_clip_rejects(vals, f):
    with pytest.raises(ValueError):
        o.teaching_clip_qdq(vals, f)


def test_clip_factors():
    f = o.clip_factors()
    assert f.dtype == np.float32 and len(f) == EX["n_candidates"]
    assert f[0] == EX["factors_first_last"][0] and f[-1] == np.float32(EX["factors_first_last"][1])
    assert np.all(np.diff(f) < 0)


# ------------------------------------------------------------------ fp32 contract
def test_quantize_clipped_hand_vector():
    """Group [-1, 0.5, 0.25, 1] (padded to 128 with copies of its values) at c = 0.75, worked in
    fp32 by hand: the clamp gives [-0.75, 0.5, 0.25, 0.75]; Delta = RN(1.5 / 15) = RN(0.1) =
    0x3DCCCCCD.  -mn / Delta = 0.75 / 0.100000001490116 = 7.4999998882..., whose nearest fp32 is
    7.5 (the neighbour below, 7.4999995, is farther), so z = rne(7.5) = 8.  The quotients are
    -7.5, 5 (4.99999992... rounds to 5), 2.5 (2.49999996... rounds to 2.5) and 7.5; rne gives
    -8, 5, 2, 8; adding z and clamping to [0, 15] gives codes 0, 13, 10, 15, i.e. the
    reconstruction Delta (q - z) = [-0.8, 0.5, 0.2, 0.7]: the low end lands below -c and the top
    is cut to 0.7."""
    v = np.array([-1.0, 0.5, 0.25, 1.0], np.float32)
    W = np.tile(v, 32)[None, :]
    q, z, d = o.quantize_clipped(W, np.ones(128, np.float32), np.array([[0.75]], np.float32))
    assert d[0, 0].view(np.uint32) == 0x3DCCCCCD
    assert z[0, 0] == 8
    assert list(q[0, :4]) == [0, 13, 10, 15]
    rec = o.dequant_scaled(q, z, d)[0, :4]
    assert np.allclose(rec, [-0.8, 0.5, 0.2, 0.7], rtol=0, atol=1e-7)


def test_factor_one_equals_unclipped_quantizer():
    rng = np.random.default_rng(0)
    W = (rng.standard_normal((16, 256)) * 0.05).astype(np.float32)
    s = (rng.random(256) + 0.5).astype(np.float32)
    cs = o.clip_thresholds(W, s)
    q0, z0, d0 = o.quantize(W, s)
    q1, z1, d1 = o.quantize_clipped(W, s, cs[0])
    assert np.array_equal(q0, q1) and np.array_equal(z0, z1) and np.array_equal(d0.view(np.uint32), d1.view(np.uint32))


def test_thresholds_are_shrunk_absmax():
    W = np.zeros((1, 128), np.float32)
    W[0, 5] = -3.0
    W[0, 9] = 2.0
    cs = o.clip_thresholds(W, np.ones(128, np.float32))
    assert cs.shape == (10, 1, 1)
    assert cs[0, 0, 0] == 3.0 and cs[9, 0, 0] == np.float32(np.float32(0.55) * np.float32(3.0))


def _exact_err(X, W, s, c, group=128):
    """err[n, g] = mean_m (sum_{k in g} X[m,k] (W - Delta (q - z) / s)[n,k])^2 in rationals."""
    q, z, d = o.quantize_clipped(W, s, c, group)
    M, K = X.shape
    N = W.shape[0]
    out = np.empty((N, K // group))
    for n in range(N):
        for g in range(K // group):
            e = [Fraction(float(W[n, k])) - Fraction(float(d[n, g])) * (int(q[n, k]) - int(z[n, g]))
                 / Fraction(float(s[k])) for k in range(g * group, (g + 1) * group)]
            tot = Fraction(0)
            for m in range(M):
                y = sum(Fraction(float(X[m, k])) * e[k - g * group] for k in range(g * group, (g + 1) * group))
                tot += y * y
            out[n, g] = float(tot / M)
    return out


def test_clip_errors_exact_rational():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((3, 256)).astype(np.float32)
    W = (rng.standard_normal((2, 256)) * 0.1).astype(np.float32)
    W[0, 3] = 0.9  # an outlier that clipping can cut
    s = (rng.random(256) + 0.5).astype(np.float32)
    res = o.clip_errors(X, W, s, n_clip=10)
    for i in (0, 4, 9):
        ex = _exact_err(X, W, s, res["thresholds"][i])
        assert np.allclose(res["err"][i], ex, rtol=1e-12, atol=0)


def test_clip_errors_scale_with_x_squared():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((8, 256)).astype(np.float32)
    W = (rng.standard_normal((4, 256)) * 0.1).astype(np.float32)
    s = np.ones(256, np.float32)
    a, b = o.clip_errors(X, W, s), o.clip_errors(2 * X, W, s)
    assert np.array_equal(4 * a["err"], b["err"])  # exact: powers of two
    assert np.array_equal(a["best"], b["best"])


def test_first_minimum_wins_ties():
    W = (np.random.default_rng(3).standard_normal((3, 128)) * 0.1).astype(np.float32)
    res = o.clip_errors(np.zeros((4, 128), np.float32), W, np.ones(128, np.float32))
    assert np.all(res["err"] == 0) and np.all(res["best"] == 0)
    assert np.array_equal(res["max_val"], res["thresholds"][0])


def test_clipping_an_unused_outlier_helps():
    """[EXPLAINER §5]: clipping gives up a group's end points for a finer step.  With the
    outlier channel's input zero, cutting it costs nothing and every other weight gains."""
    rng = np.random.default_rng(4)
    W = rng.uniform(-0.3, 0.3, (1, 128)).astype(np.float32)
    W[0, 0] = 1.0
    X = rng.standard_normal((64, 128)).astype(np.float32)
    X[:, 0] = 0.0
    res = o.clip_errors(X, W, np.ones(128, np.float32))
    b = res["best"][0, 0]
    assert b >= 1 and res["err"][b, 0, 0] <= 0.8 * res["err"][0, 0, 0]


def test_pack_clipped():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((8, 256)) * 0.05).astype(np.float32)
    s = (rng.random(256) + 0.5).astype(np.float32)
    cs = o.clip_thresholds(W, s)
    same = o.pack_clipped(W, s, cs[0])
    plain = o.pack(W, s)
    for k in ("qweight", "scales", "zeros"):
        assert np.array_equal(same[k], plain[k])
    art = o.pack_clipped(W, s, cs[5])
    assert np.array_equal(o.unpack_words(art["qweight"]), art["codes"])
    with pytest.raises(ValueError):
        o.pack_clipped(W, s, -cs[5])
