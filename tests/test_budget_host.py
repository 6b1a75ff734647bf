"""The library's speculation-budget planner (host code in libprr.so, no GPU) against the oracle: the same
coefficients to float64 rounding, the same choice wherever the decision is not a float64 near-tie, the
table rows read as they are, and every invalid table rejected before anything is written."""
import ctypes

import numpy as np
import pytest

from block_sparse_attention_quest_amd import binding as bd
from oracle import prr_oracle as O

CTX = np.array([4096.0, 8192.0, 16384.0, 32768.0, 65536.0])
DELTAS = np.array([0.25, 0.5, 0.75, 1.0, 1.5, 2.0, 3.0, 4.0])


def _table(seed):
    """Latency-shaped synthetic profiles: selection grows about linearly with context, speculative
    attention grows with delta and slightly with context; multiplicative noise."""
    rng = np.random.default_rng(seed)
    sel = (3.0 + 0.25 * CTX / 1024.0) * rng.uniform(0.9, 1.1, size=CTX.size)
    spec = np.array([(2.0 + 9.0 * d + 0.01 * CTX / 1024.0) * rng.uniform(0.9, 1.1, size=CTX.size) for d in DELTAS])
    return sel, spec


@pytest.mark.parametrize("degree", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_library_fit_and_choice_match_the_oracle(degree, seed):
    sel, spec = _table(seed)
    tab = bd.BudgetTable(CTX, sel, DELTAS, spec, degree)
    want = O.budget_fit(CTX, sel, DELTAS, spec, degree)
    scale = max(1.0, np.abs(want).max())
    np.testing.assert_allclose(tab.coef, want, rtol=0, atol=1e-9 * scale)
    for T in [2048.0, 4096.0, 6000.0, 24576.0, 65536.0, 131072.0, 262144.0, 524288.0]:
        j, est = tab.choose(T)
        wj, west = O.budget_choose(CTX, sel, DELTAS, spec, want, T)
        np.testing.assert_allclose(est, west, rtol=1e-9, atol=1e-9 * scale)
        margins = np.abs(west[1:] - west[0])
        if margins.min() > 1e-6 * scale:   # away from a float64 near-tie the decision is unique
            assert j == wj, (T, est, west)


def test_profiled_length_reads_the_table_bit_for_bit():
    sel, spec = _table(7)
    tab = bd.BudgetTable(CTX, sel, DELTAS, spec, 2)
    for i, T in enumerate(CTX):
        j, est = tab.choose(T)
        assert est.tolist() == [sel[i]] + spec[:, i].tolist()
        fits = [k for k in range(DELTAS.size) if spec[k, i] <= sel[i]]
        assert j == (max(fits) if fits else -1)


def test_hand_table_choices():
    ctx, sel, deltas = [4096.0, 8192.0, 16384.0], [10.0, 20.0, 40.0], [0.5, 1.0, 2.0]
    spec = [[5.0, 5.0, 5.0], [9.0, 12.0, 15.0], [18.0, 20.0, 30.0]]
    tab = bd.BudgetTable(ctx, sel, deltas, spec, 1)
    assert [tab.choose(T)[0] for T in (4096.0, 8192.0, 16384.0, 12288.0)] == [1, 2, 2, 2]
    none = bd.BudgetTable(ctx, [1.0, 1.0, 1.0], [1.0], [[2.0, 2.0, 2.0]], 1)
    assert none.choose(6000.0)[0] == -1


def _call_fit(ctx, sel, deltas, spec, degree, coef):
    lib = bd.load_library()
    a = [np.ascontiguousarray(v, dtype=np.float64) for v in (ctx, sel, deltas, spec)]
    return lib.prr_budget_fit(a[0].ctypes.data, len(a[0]), a[1].ctypes.data, a[2].ctypes.data, len(a[2]),
                              a[3].ctypes.data, degree, coef.ctypes.data if coef is not None else None)


@pytest.mark.parametrize("case", ["degree_high", "degree_neg", "ctx_unsorted", "ctx_zero", "delta_dup",
                                  "delta_neg", "nan_time", "inf_ctx", "null_coef", "too_many"])
def test_invalid_tables_are_rejected_and_nothing_is_written(case):
    ctx, sel = CTX.copy(), np.ones(CTX.size)
    deltas, spec, degree = DELTAS.copy(), np.ones((DELTAS.size, CTX.size)), 2
    coef = np.full((1 + DELTAS.size, 5), 7.0)
    if case == "degree_high":
        degree = 5
    elif case == "degree_neg":
        degree = -1
    elif case == "ctx_unsorted":
        ctx[[1, 2]] = ctx[[2, 1]]
    elif case == "ctx_zero":
        ctx[0] = 0.0
    elif case == "delta_dup":
        deltas[3] = deltas[2]
    elif case == "delta_neg":
        deltas[0] = -0.25
    elif case == "nan_time":
        spec[2, 3] = np.nan
    elif case == "inf_ctx":
        ctx[-1] = np.inf
    elif case == "too_many":
        ctx = np.arange(1, 66, dtype=np.float64)
        sel, spec = np.ones(65), np.ones((DELTAS.size, 65))
    st = _call_fit(ctx, sel, deltas, spec, degree, None if case == "null_coef" else coef)
    assert st == 1   # PRR_EINVAL
    assert (coef == 7.0).all()


def test_degree_above_the_points_is_rejected_and_choose_checks_context():
    lib = bd.load_library()
    coef = np.zeros((2, 3))
    assert _call_fit([1.0, 2.0], [1.0, 2.0], [1.0], [[1.0, 1.0]], 2, coef) == 1
    tab = bd.BudgetTable([1.0, 2.0], [1.0, 2.0], [1.0], [[1.0, 1.0]], 1)
    choice = ctypes.c_int32(5)
    for bad in (0.0, -3.0, float("nan"), float("inf")):
        st = lib.prr_budget_choose(*tab._table(), tab.coef.ctypes.data, bad, ctypes.addressof(choice), None, 0, None)
        assert st == 1 and choice.value == 5
    # est is optional
    assert lib.prr_budget_choose(*tab._table(), tab.coef.ctypes.data, 1.5, ctypes.addressof(choice), None, 0,
                                 None) == 0
    assert choice.value == 0
    # a negative top-K is refused when |P| is asked for
    blocks = ctypes.c_int32(7)
    assert lib.prr_budget_choose(*tab._table(), tab.coef.ctypes.data, 1.5, ctypes.addressof(choice), None, -1,
                                 ctypes.addressof(blocks)) == 1 and blocks.value == 7


def test_speculation_budget_blocks():
    from block_sparse_attention_quest_amd.layer_step import speculation_budget

    ctx, sel, deltas = [4096.0, 8192.0, 16384.0], [10.0, 20.0, 40.0], [0.5, 1.0, 2.0]
    spec = [[5.0, 5.0, 5.0], [9.0, 12.0, 15.0], [18.0, 20.0, 30.0]]
    tab = bd.BudgetTable(ctx, sel, deltas, spec, 1)
    assert speculation_budget(tab, 4096, 64) == 64      # delta 1
    assert speculation_budget(tab, 16384, 64) == 128    # delta 2
    slow = bd.BudgetTable(ctx, [1.0, 1.0, 1.0], deltas, spec, 1)
    assert speculation_budget(slow, 8192, 64) == 32     # nothing fits: the smallest delta
    assert speculation_budget(slow, 8192, 1) == 0       # |P| <= 0.5 |A| = 0.5 admits no block


def test_budget_blocks_match_the_oracle():
    """|P| in blocks from the C ABI against the oracle's budget_blocks over random tables, lengths (on and
    off the grid) and top-K sizes, with ratios whose products land near integers."""
    rng = np.random.default_rng(17)
    ctx = [4096.0, 8192.0, 16384.0, 32768.0]
    deltas = [0.0, 0.29, 0.7, 1.0, 1.25, 2.5]
    for _ in range(40):
        sel = np.sort(rng.uniform(5, 60, size=4))
        spec = np.sort(rng.uniform(2, 80, size=(len(deltas), 1)), axis=0) + rng.uniform(0, 5, size=(len(deltas), 4))
        tab = bd.BudgetTable(ctx, sel, deltas, spec, 1)
        coef = O.budget_fit(ctx, sel, deltas, spec, 1)
        for T in (4096.0, 12000.0, 32768.0, 50000.0):
            for k in (0, 1, 3, 64, 100, 257):
                j, _ = O.budget_choose(ctx, sel, deltas, spec, coef, T)
                assert tab.budget_blocks(T, k) == O.budget_blocks(deltas, j, k), (T, k, j)
