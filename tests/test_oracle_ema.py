"""Pins for the oracle's EMA predictor and calibration (CPU only).

Independent facts ([paper] §4.1 prediction/update; [blog] Eqs. (2)-(3); [paper] §4.2 and [blog]
Eqs. (4)-(5) for calibration):
  * hand-worked steps (tests/golden/ema_hand_steps.json) and a hand-worked calibration
    (tests/golden/calibration_hand.json), derived on paper from the equations;
  * alpha = 1, gamma = 0 reproduces "reuse the previous top-K" ([paper] §5.3 ablation S1);
  * a constant score is a fixed point; a linear ramp a + b t converges to trend b/alpha and a
    prediction error b (gamma - 1)/alpha (derived from the two recurrences);
  * calibration: H in [0, 1]; constant rows give H = 1; K >= N gives H = 1; the grid is the
    4 x 5 x 4 = 80 points the pages list.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import prr_oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_hand_worked_steps():
    for case in _load("ema_hand_steps.json")["cases"]:
        a, b, g = case["alpha"], case["beta"], case["gamma"]
        IS = case["IS"]
        level = np.array([IS[0]])
        trend = np.zeros(1)
        # step 0: the block is born
        lv, tr, live, _ = orc.predict_step(np.zeros(0), np.zeros(0), 0, np.array([IS[0]]), a, b, g, 1)
        assert lv[0] == case["level"][0] and tr[0] == case["trend"][0] and live == 1
        level, trend = lv, tr
        for t in range(1, len(IS)):
            assert orc.ema_predict(level, trend, g)[0] == case["pred"][t - 1]
            level, trend = orc.ema_update(level, trend, np.array([IS[t]]), a, b)
            assert level[0] == case["level"][t] and trend[0] == case["trend"][t]
        assert orc.ema_predict(level, trend, g)[0] == case["pred"][-1]


def test_reuse_previous_topk_special_case():
    """alpha = 1, gamma = 0: the prediction is last step's scores, so P^t = A^{t-1}."""
    rng = np.random.default_rng(7)
    n, k = 60, 9
    IS = rng.standard_normal((6, n))
    lv, tr, live, P = orc.predict_step(np.zeros(0), np.zeros(0), 0, IS[0], 1.0, 0.4, 0.0, k)
    for t in range(1, 6):
        assert list(P) == list(orc.topk_blocks(IS[t - 1], k))
        lv, tr, live, P = orc.predict_step(lv, tr, live, IS[t], 1.0, 0.4, 0.0, k)


def test_constant_scores_fixed_point():
    IS = np.array([3.5, -1.25, 7.0])
    lv, tr, live, _ = orc.predict_step(np.zeros(0), np.zeros(0), 0, IS, 0.3, 0.7, 0.6, 2)
    for _ in range(20):
        lv, tr, live, _ = orc.predict_step(lv, tr, live, IS, 0.3, 0.7, 0.6, 2)
    assert np.array_equal(lv, IS) and np.array_equal(tr, np.zeros(3))


@pytest.mark.parametrize("alpha,beta,gamma", [(0.6, 0.3, 0.5), (0.2, 0.1, 0.0), (0.8, 0.5, 0.75)])
def test_ramp_asymptotics(alpha, beta, gamma):
    a, b = 2.0, 0.125
    lv, tr, live, _ = orc.predict_step(np.zeros(0), np.zeros(0), 0, np.array([a]), alpha, beta,
                                       gamma, 1)
    for t in range(1, 400):
        pred = orc.ema_predict(lv, tr, gamma)[0]
        lv, tr, live, _ = orc.predict_step(lv, tr, live, np.array([a + b * t]), alpha, beta, gamma, 1)
    assert abs(tr[0] - b / alpha) < 1e-9
    assert abs((pred - (a + b * 399)) - b * (gamma - 1) / alpha) < 1e-9


def test_births_join_with_their_score():
    lv, tr, live, _ = orc.predict_step(np.zeros(0), np.zeros(0), 0, np.array([1.0, 2.0]), 0.5, 0.5,
                                       0.5, 1)
    lv, tr, live, P = orc.predict_step(lv, tr, live, np.array([3.0, 2.0, 9.0]), 0.5, 0.5, 0.5, 2)
    assert live == 3 and lv[2] == 9.0 and tr[2] == 0.0
    assert list(P) == [0, 2]   # predictions [2+0.5*1, 2, 9]


def test_calibration_hand_worked():
    g = _load("calibration_hand.json")
    H, best = orc.calibrate(np.array(g["IS"]), g["k"], np.array(g["grid"]))
    for h, (num, den) in zip(H, g["H_num_den"]):
        assert abs(h - num / den) < 1e-15
    assert best == g["best"]
    assert Fraction(26, 45) > Fraction(137, 315)


def test_calibration_grid_is_the_pages_grid():
    grid = orc.calibration_grid()
    assert grid.shape == (80, 3)
    assert sorted(set(grid[:, 0])) == [0.2, 0.4, 0.6, 0.8]
    assert sorted(set(grid[:, 1])) == [0.1, 0.2, 0.3, 0.4, 0.5]
    assert sorted(set(grid[:, 2])) == [0.0, 0.25, 0.5, 0.75]
    assert list(grid[0]) == [0.2, 0.1, 0.0] and list(grid[1]) == [0.2, 0.1, 0.25]
    assert list(grid[4]) == [0.2, 0.2, 0.0] and list(grid[20]) == [0.4, 0.1, 0.0]


def test_calibration_sanity():
    rng = np.random.default_rng(9)
    const = np.tile(rng.random(12) + 0.5, (10, 1))
    H, best = orc.calibrate(const, 4)
    assert np.all(H == 1.0) and best == 0
    H, _ = orc.calibrate(rng.random((15, 6)) + 0.1, 6)      # K >= N: P = A = everything
    assert np.all(H == 1.0)
    IS = np.exp(rng.standard_normal((40, 20)))
    H, best = orc.calibrate(IS, 5)
    assert np.all(H >= 0.0) and np.all(H <= 1.0) and H[best] == H.max()
    assert best == int(np.flatnonzero(H == H.max())[0])


def test_crossing_ramps_favour_fast_tracking():
    """Blocks whose scores rise and fall linearly: a predictor that follows the level quickly and
    extrapolates the trend (large alpha, large gamma) wins; the steady-state ranking coefficient of a
    slope b is b (gamma - 1 + alpha)/alpha (from the ramp asymptotics)."""
    T, n = 200, 16
    rng = np.random.default_rng(3)
    slopes = rng.choice([-1.0, 1.0], size=n) * rng.uniform(0.05, 0.2, size=n)
    phase = rng.uniform(0, T, size=n)
    t = np.arange(T)[:, None]
    IS = 10.0 + np.abs(((t - phase) * slopes) % 8.0 - 4.0)   # triangle waves, positive
    H, best = orc.calibrate(IS, 4)
    a, b, g = orc.calibration_grid()[best]
    assert a == 0.8 and g == 0.75
