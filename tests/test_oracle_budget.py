"""Pins of the oracle's speculation-budget planner ([paper] §4.4, A.6): the least-squares polynomial
against closed forms and the normal equations, the table lookup at profiled lengths, and the choice rule
on hand-worked tables."""
import numpy as np
import pytest

from oracle import prr_oracle as O

CTX = [4096.0, 8192.0, 16384.0, 32768.0, 65536.0]


def _x():
    return np.array(CTX) / CTX[-1]


@pytest.mark.parametrize("degree", [0, 1, 2, 3, 4])
def test_fit_recovers_an_exact_polynomial(degree):
    rng = np.random.default_rng(11 + degree)
    c = rng.normal(size=degree + 1) * 10
    y = np.array([sum(ck * x ** k for k, ck in enumerate(c)) for x in _x()])
    coef = O.budget_fit(CTX, y, [1.0], [y], degree)
    np.testing.assert_allclose(coef[0], c, rtol=0, atol=1e-8 * max(1.0, np.abs(c).max()))
    np.testing.assert_allclose(coef[1], c, rtol=0, atol=1e-8 * max(1.0, np.abs(c).max()))


def test_degree_zero_is_the_mean_and_degree_one_the_textbook_line():
    y = np.array([3.0, 5.5, 4.0, 9.0, 12.25])
    assert O.budget_fit(CTX, y, [1.0], [y], 0)[0][0] == pytest.approx(y.mean(), rel=1e-14)
    x = _x()
    slope = ((x - x.mean()) * (y - y.mean())).sum() / ((x - x.mean()) ** 2).sum()
    icpt = y.mean() - slope * x.mean()
    np.testing.assert_allclose(O.budget_fit(CTX, y, [1.0], [y], 1)[0], [icpt, slope], rtol=1e-12)


@pytest.mark.parametrize("degree", [1, 2, 3])
def test_residual_is_orthogonal_to_every_column(degree):
    # the least-squares optimum satisfies the normal equations V^T (y - V c) = 0
    rng = np.random.default_rng(5)
    y = rng.uniform(5, 50, size=len(CTX))
    c = O.budget_fit(CTX, y, [0.5], [y * 0.3], degree)[0]
    V = np.vander(_x(), degree + 1, increasing=True)
    r = y - V @ c
    assert np.abs(V.T @ r).max() <= 1e-10 * np.abs(y).max()


def test_as_many_points_as_coefficients_interpolates():
    y = np.array([7.0, 1.0, 4.0, 9.0, 2.0])
    c = O.budget_fit(CTX, y, [1.0], [y], 4)[0]
    fit = np.array([sum(ck * x ** k for k, ck in enumerate(c)) for x in _x()])
    np.testing.assert_allclose(fit, y, rtol=0, atol=1e-9)


# A hand-worked table: three lengths, three budget ratios.
#   selection:       10   20   40
#   delta 0.5 spec:   5    5    5
#   delta 1.0 spec:   9   12   15
#   delta 2.0 spec:  18   20   30
# At 4096 tokens delta 1 (9 <= 10) fits and delta 2 (18 > 10) does not -> index 1.  At 8192 delta 2
# spends exactly the window (20 <= 20) -> index 2.  At 16384 all fit -> index 2.
HAND_CTX = [4096.0, 8192.0, 16384.0]
HAND_SEL = [10.0, 20.0, 40.0]
HAND_DELTAS = [0.5, 1.0, 2.0]
HAND_SPEC = [[5.0, 5.0, 5.0], [9.0, 12.0, 15.0], [18.0, 20.0, 30.0]]


@pytest.mark.parametrize("context,want", [(4096.0, 1), (8192.0, 2), (16384.0, 2)])
def test_choice_on_the_hand_table(context, want):
    coef = O.budget_fit(HAND_CTX, HAND_SEL, HAND_DELTAS, HAND_SPEC, 1)
    j, est = O.budget_choose(HAND_CTX, HAND_SEL, HAND_DELTAS, HAND_SPEC, coef, context)
    assert j == want
    i = HAND_CTX.index(context)    # a profiled length reads the table, not the fit
    assert est.tolist() == [HAND_SEL[i]] + [r[i] for r in HAND_SPEC]


def test_off_grid_length_reads_the_line():
    # at x = T / 16384 the selection row (0.25, 10), (0.5, 20), (1, 40) is exactly 40 x, so 12288 tokens
    # (x = 0.75) estimate 30; the flat delta-0.5 row estimates 5 there
    coef = O.budget_fit(HAND_CTX, HAND_SEL, HAND_DELTAS, HAND_SPEC, 1)
    np.testing.assert_allclose(coef[0], [0.0, 40.0], atol=1e-12)
    j, est = O.budget_choose(HAND_CTX, HAND_SEL, HAND_DELTAS, HAND_SPEC, coef, 12288.0)
    assert est[0] == pytest.approx(30.0, abs=1e-12)
    assert est[1] == pytest.approx(5.0, abs=1e-12)
    # delta 2 row (0.25, 18), (0.5, 20), (1, 30): xbar = 7/12, ybar = 68/3, Sxy = 29/6, Sxx = 7/24, so
    # the line's slope is 116/7 and its value at 0.75 is 68/3 + (116/7)(1/6), about 25.43 <= 30
    assert est[3] == pytest.approx(68.0 / 3.0 + (116.0 / 7.0) / 6.0, abs=1e-9)
    assert j == 2


def test_no_fitting_ratio_gives_minus_one_and_delta_zero_always_fits():
    sel = [1.0, 1.0, 1.0]
    spec = [[2.0, 2.0, 2.0]]
    coef = O.budget_fit(HAND_CTX, sel, [1.0], spec, 1)
    assert O.budget_choose(HAND_CTX, sel, [1.0], spec, coef, 6000.0)[0] == -1
    spec0 = [[0.0, 0.0, 0.0], [2.0, 2.0, 2.0]]
    coef = O.budget_fit(HAND_CTX, sel, [0.0, 1.0], spec0, 1)
    assert O.budget_choose(HAND_CTX, sel, [0.0, 1.0], spec0, coef, 6000.0)[0] == 0


def test_longer_selection_never_lowers_the_choice():
    # with speculative latency increasing in delta, a larger selection window can only admit more
    rng = np.random.default_rng(3)
    for _ in range(50):
        spec = np.sort(rng.uniform(1, 40, size=(6, 1)), axis=0)
        last = -2
        for s in np.linspace(0, 45, 31):
            j, _ = O.budget_choose([4096.0], [s], list(range(6)), spec, np.zeros((7, 1)), 4096.0)
            assert j >= last
            last = j


@pytest.mark.parametrize("deltas,choice,topk,want", [
    ([0.5, 1.0, 2.0], 1, 64, 64),        # delta 1: |P| = K
    ([0.5, 1.0, 2.0], 2, 64, 128),       # delta 2
    ([0.75], 0, 2, 1),                   # 1.5 blocks allowed: |P| <= delta |A| admits 1, not 2
    ([0.25, 1.5], 1, 3, 4),              # 4.5 -> 4
    ([0.5, 1.0], -1, 64, 32),            # nothing fits: the smallest profiled ratio
    ([0.0, 1.0], 0, 64, 0),              # delta 0: no speculation
    ([0.29], 0, 100, 29),                # 0.29 * 100 rounds to 28.999999999999996 in float64
    ([0.7], 0, 10, 7),                   # 7.000000000000001
    ([1.0], 0, 0, 0),                    # K = 0: |A| = 0
])
def test_budget_blocks_is_the_largest_set_the_constraint_admits(deltas, choice, topk, want):
    """[blog] Eq. (1): |P| <= delta |A|; the largest admissible |P| is floor(delta K)."""
    assert O.budget_blocks(deltas, choice, topk) == want
