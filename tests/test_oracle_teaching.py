"""Pins the oracle's teaching mode, scale family and argmin to the values the AWQ explainer
page prints for its two-channel worked example (tests/golden/explainer_worked_examples.json)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import awq_oracle as o
from tests.conftest import GOLDEN

G = json.load(open(os.path.join(GOLDEN, "explainer_worked_examples.json"), encoding="utf-8"))


@pytest.mark.parametrize("case", G["hand_picked"])
def test_hand_picked_scales(case):
    y, codes, step = o.teaching_forward(G["x"], G["w"], case["scales"])
    assert math.isclose(y, case["y_num"] / case["y_den"], abs_tol=1e-12)
    if "codes" in case:
        assert codes == case["codes"]
    if "step_num" in case:
        assert math.isclose(step, case["step_num"] / case["step_den"], rel_tol=1e-15)
    if "restored_num" in case:
        _, restored, _ = o.teaching_qdq([wi * si for wi, si in zip(G["w"], case["scales"])])
        want = [n / d for n, d in case["restored_num"]]
        assert all(math.isclose(r, v, rel_tol=1e-15) for r, v in zip(restored, want))


def test_twenty_candidate_search_matches_page():
    r = o.teaching_search(G["x"], G["w"])
    best = r["best"]
    s = G["search"]
    assert len(r["y"]) == len(r["loss"]) == len(r["alpha"]) == s["n_candidates"]
    assert r["target"] == G["target"]["value"]
    assert r["alpha"][-1] == s["last_alpha"]
    assert r["alpha"][best] == s["alpha_best"]
    assert round(r["y"][best], s["printed_decimals"]) == s["y_best_printed"]
    # the chosen candidate beats the unscaled one (alpha = 0)
    assert r["loss"][best] < r["loss"][0]
    # alpha = 0 is the unscaled layer: y = 17/7, loss (17/7 - 2)^2 = 9/49
    assert math.isclose(r["loss"][0], 9 / 49, rel_tol=1e-12)
    assert math.isclose(r["y"][0], 17 / 7, rel_tol=1e-15)


def test_alpha_grid_excludes_one():
    g = o.alpha_grid()
    assert len(g) == 20 and g[0] == 0.0 and g[-1] == 0.95 and 1.0 not in g
    assert all(math.isclose(b - a, 0.05, abs_tol=1e-12) for a, b in zip(g, g[1:]))


@pytest.mark.parametrize("chk", G["quantizer_checks"])
def test_teaching_quantizer_checks(chk):
    codes, restored, step = o.teaching_qdq(chk["values"])
    assert codes == chk["codes"]
    if "restored" in chk:
        assert restored == chk["restored"] and step == chk["step"]


def test_common_scale_gives_no_gain():
    c = G["common_scales"]
    for v in c["values"]:
        y, _, _ = o.teaching_forward(G["x"], G["w"], [v, v])
        assert math.isclose(y, c["y_num"] / c["y_den"], abs_tol=1e-12)


@pytest.mark.parametrize("bad", [[float("nan")], [float("inf"), 1.0], []])
def test_teaching_rejects_nonfinite(bad):
    with pytest.raises(ValueError):
        o.teaching_qdq(bad)


@pytest.mark.parametrize("x,w,s", [
    ([1.0], [1.0, 2.0], [1.0, 1.0]),          # length mismatch
    ([1.0, 2.0], [1.0, 2.0], [1.0, 0.0]),     # non-positive scale
    ([1.0, 2.0], [1.0, 2.0], [1.0, -1.0]),
    ([1e-300, 1.0], [1.0, 1.0], [1e300, 1.0]),  # x / s underflows to zero
    ([float("nan"), 1.0], [1.0, 1.0], [1.0, 1.0]),
])
def test_teaching_forward_range_checks(x, w, s):
    with pytest.raises(ValueError):
        o.teaching_forward(x, w, s)


def test_exact_rational_y_for_chosen_candidate():
    # y at the chosen alpha recomputed in exact rationals from the quantizer's definition
    # (codes from nearest rounding, step = max|v|/7) agrees with the float search.
    r = o.teaching_search(G["x"], G["w"])
    alpha = float(r["alpha"][r["best"]])
    s = [Fraction(float(v)) for v in o.candidate_scales([abs(v) for v in G["x"]], alpha)]
    x = [Fraction(v) for v in G["x"]]
    w = [Fraction(v) for v in G["w"]]
    ws = [a * b for a, b in zip(w, s)]
    step = max(abs(v) for v in ws) / 7
    codes = [min(7, max(-7, round(v / step))) for v in ws]
    y = sum(xi / si * step * c for xi, si, c in zip(x, s, codes))
    assert abs(float(y) - r["y"][r["best"]]) < 1e-12


def test_bits_per_weight_budget():
    b = G["bits_per_weight"]
    assert o.artefact_bits_per_weight(4096, 4096, b["group"]) == b["value"]
    assert round(16 / b["value"], 2) == b["ratio_vs_16bit"]
