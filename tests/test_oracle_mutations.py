"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in the oracle (on the CPU, via monkeypatch: a dropped term, a wrong sign or
index, a transposed operand, a swapped coefficient) and runs the pins that should notice it; the case
passes only if at least one of those pins fails.
"""
import math

import numpy as np
import pytest

import test_oracle_attention as ta
import test_oracle_budget as tb
import test_oracle_ema as te
import test_oracle_fp8 as tf
import test_oracle_mean as tm
import test_oracle_select as ts
from _util import oracle_view
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

_orig = {name: getattr(orc, name) for name in dir(orc) if callable(getattr(orc, name))}


def _small_fixture(w):
    q, kv = oracle_view(wl.make_inputs(w))
    return w, q[0], kv


def _sel_fixture():
    q, kv = oracle_view(wl.make_inputs(ts.W))
    return q[0], kv, orc.build_meta(kv, ts.W.block, ts.W.num_kv_heads)


def _fails(*checks):
    for fn, args in checks:
        try:
            fn(*args)
        except AssertionError:
            return True
    return False


# ---- planted mistakes ----

def merge_wrong_sign(a, b):
    m = max(a.m, b.m)
    if m == -math.inf:
        return orc.State(a.acc + b.acc, 0.0, -math.inf)
    fa = 0.0 if a.m == -math.inf else math.exp(m - a.m)
    fb = 0.0 if b.m == -math.inf else math.exp(b.m - m)
    return orc.State(fa * a.acc + fb * b.acc, fa * a.l + fb * b.l, m)


def merge_drop_l_term(a, b):
    s = _orig["merge"](a, b)
    fa = 0.0 if a.m == -math.inf else math.exp(a.m - s.m) if s.m != -math.inf else 0.0
    return orc.State(s.acc, fa * a.l, s.m)


def gather_v_is_k(kv, b, kvh, blocks, block):
    K, _ = _orig["gather_kv"](kv, b, kvh, blocks, block)
    return K, K.copy()


def gather_v_wrong_token(kv, b, kvh, blocks, block):
    K, V = _orig["gather_kv"](kv, b, kvh, blocks, block)
    return K, V[::-1].copy()


def quest_max_only(qbar, mn, mx):
    s = np.zeros(mn.shape[0])
    for i in range(mn.shape[1]):
        s = s + qbar[i] * mx[:, i]
    return s


def rep_query_no_divide(q_all, b, kvh, G):
    return _orig["representative_query"](q_all, b, kvh, G) * G


def rep_query_wrong_heads(q_all, b, kvh, G):
    return np.mean(q_all[b, kvh::max(1, q_all.shape[1] // G)][:G], axis=0)


def topk_ties_to_larger(scores, k):
    n = scores.shape[0]
    k = max(0, min(int(k), n))
    order = np.lexsort((-np.arange(n), -scores))
    return np.sort(order[:k]).astype(np.int64)


def ema_trend_uses_new_level(level, trend, IS, alpha, beta):
    new_level = alpha * IS + (1.0 - alpha) * level
    new_trend = beta * (IS - new_level) + (1.0 - beta) * trend
    return new_level, new_trend


def ema_swapped_alpha(level, trend, IS, alpha, beta):
    new_trend = beta * (IS - level) + (1.0 - beta) * trend
    new_level = (1.0 - alpha) * IS + alpha * level
    return new_level, new_trend


def ema_predict_minus(level, trend, gamma):
    return level - gamma * trend


def hit_rate_unweighted(IS_row, P, A):
    return len(np.intersect1d(P, A)) / max(1, len(A))


def calibrate_divide_by_T(IS, k, grid=None):
    H, best = _orig["calibrate"](IS, k, grid)
    T = np.asarray(IS).shape[0]
    return H * (T - 1) / T, best


def mean_divides_by_block_size(kv, b, kvh, p, block):
    K, _ = orc.gather_kv(kv, b, kvh, [p], block)
    acc = np.zeros(K.shape[1])
    for t in range(K.shape[0]):
        acc = acc + K[t]
    return (acc / block).astype(np.float32).astype(np.float64)


def mean_scores_abs(qbar, mean):
    s = np.zeros(mean.shape[0])
    for i in range(mean.shape[1]):
        s = s + abs(qbar[i]) * mean[:, i]
    return s


def mean_skips_first_token(kv, b, kvh, p, block):
    K, _ = orc.gather_kv(kv, b, kvh, [p], block)
    K = K[1:] if K.shape[0] > 1 else K
    return (K.sum(axis=0) / K.shape[0]).astype(np.float32).astype(np.float64)


def fp8_bias_8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -10, (1.0 + m / 8.0) * np.exp2((e - 8).astype(np.float64)))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def fp8_subnormals_flushed(codes):
    v = _orig["fp8_e4m3_decode"](codes)
    e = (np.asarray(codes, dtype=np.uint8) >> 3) & 0xF
    return np.where(e == 0, 0.0 * v, v)


def fp8_no_nan(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e, m = (c >> 3) & 0xF, c & 0x7
    return sign * np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))


def budget_fit_unscaled_x(ctx, t_select, deltas, t_spec, degree):
    V = np.vander(np.asarray(ctx, dtype=np.float64), degree + 1, increasing=True)
    rows = [np.asarray(t_select, dtype=np.float64)] + [np.asarray(r, dtype=np.float64) for r in t_spec]
    return np.array([np.linalg.lstsq(V, y, rcond=None)[0] for y in rows])


def budget_fit_drops_top_power(ctx, t_select, deltas, t_spec, degree):
    c = _orig["budget_fit"](ctx, t_select, deltas, t_spec, max(0, degree - 1))
    return np.concatenate([c, np.zeros((c.shape[0], degree + 1 - c.shape[1]))], axis=1)


def budget_estimates_never_read_table(ctx, t_select, t_spec, coef, context):
    x = float(context) / float(ctx[-1])
    return np.array([sum(c * x ** k for k, c in enumerate(row)) for row in coef])


def budget_estimates_scaled_by_shortest(ctx, t_select, t_spec, coef, context):
    if float(context) in [float(c) for c in ctx]:
        return _orig["budget_estimates"](ctx, t_select, t_spec, coef, context)
    x = float(context) / float(ctx[0])
    return np.array([sum(c * x ** k for k, c in enumerate(row)) for row in coef])


def budget_choose_strict(ctx, t_select, deltas, t_spec, coef, context):
    est = orc.budget_estimates(ctx, t_select, t_spec, coef, context)
    fits = [j for j in range(len(deltas)) if est[1 + j] < est[0]]
    return (max(fits) if fits else -1), est


def budget_choose_smallest(ctx, t_select, deltas, t_spec, coef, context):
    est = orc.budget_estimates(ctx, t_select, t_spec, coef, context)
    fits = [j for j in range(len(deltas)) if est[1 + j] <= est[0]]
    return (min(fits) if fits else -1), est


def budget_blocks_rounded(deltas, choice, topk):
    return int(round(float(deltas[choice if choice >= 0 else 0]) * topk))


def budget_blocks_no_slack(deltas, choice, topk):
    return int(np.floor(float(deltas[choice if choice >= 0 else 0]) * topk))


def budget_blocks_largest_fallback(deltas, choice, topk):
    d = float(deltas[choice if choice >= 0 else -1])
    x = d * topk
    return int(np.floor(x + 1e-9 * max(1.0, x)))


def _budget_checks():
    hand = [(tb.test_choice_on_the_hand_table, (c, w)) for c, w in [(4096.0, 1), (8192.0, 2), (16384.0, 2)]]
    return [(tb.test_fit_recovers_an_exact_polynomial, (2,)), (tb.test_degree_zero_is_the_mean_and_degree_one_the_textbook_line, ()),
            (tb.test_residual_is_orthogonal_to_every_column, (2,)), (tb.test_as_many_points_as_coefficients_interpolates, ()),
            *hand, (tb.test_off_grid_length_reads_the_line, ()),
            (tb.test_no_fitting_ratio_gives_minus_one_and_delta_zero_always_fits, ()),
            (tb.test_longer_selection_never_lowers_the_choice, ()),
            *[(tb.test_budget_blocks_is_the_largest_set_the_constraint_admits, c) for c in (
                ([0.75], 0, 2, 1), ([0.25, 1.5], 1, 3, 4), ([0.5, 1.0], -1, 64, 32), ([0.29], 0, 100, 29))]]


def _fp8_checks():
    return [(tf.test_decode_matches_torch_float8_e4m3fn, ()), (tf.test_known_codes, ()),
            (tf.test_positive_codes_increase_and_negatives_mirror, ())]


def _mean_checks():
    q, kv = oracle_view(wl.make_inputs(tm.W))
    fxm = (q[0], kv, orc.build_meta(kv, tm.W.block, tm.W.num_kv_heads),
           orc.build_mean_meta(kv, tm.W.block, tm.W.num_kv_heads))
    return [(tm.test_mean_matches_numpy_mean, (fxm,)), (tm.test_mean_score_bounded_by_quest_score, (fxm,)),
            (tm.test_identical_keys_and_partial_blocks, ()), (tm.test_single_token_blocks_score_is_dot_product, ())]


def _attention_checks():
    fx = _small_fixture(ta.SMALL)
    return [(ta.test_decomposition_identity, (fx,)), (ta.test_dense_case_matches_torch_sdpa, (fx,)),
            (ta.test_closed_forms, ())]


def _select_checks():
    sel = _sel_fixture()
    return [(ts.test_quest_score_is_upper_bound, (sel,)), (ts.test_representative_query_is_group_mean, (sel,)),
            (ts.test_planted_blocks_are_selected, ()), (ts.test_topk_matches_heapq_with_ties, ())]


def _ema_checks():
    return [(te.test_hand_worked_steps, ()), (te.test_calibration_hand_worked, ()),
            (te.test_ramp_asymptotics, (0.6, 0.3, 0.5))]


MUTATIONS = [
    ("merge", merge_wrong_sign, _attention_checks),
    ("merge", merge_drop_l_term, _attention_checks),
    ("gather_kv", gather_v_is_k, _attention_checks),
    ("gather_kv", gather_v_wrong_token, _attention_checks),
    ("quest_scores", quest_max_only, _select_checks),
    ("representative_query", rep_query_no_divide, _select_checks),
    ("representative_query", rep_query_wrong_heads, _select_checks),
    ("topk_blocks", topk_ties_to_larger, _select_checks),
    ("ema_update", ema_trend_uses_new_level, _ema_checks),
    ("ema_update", ema_swapped_alpha, _ema_checks),
    ("ema_predict", ema_predict_minus, _ema_checks),
    ("hit_rate_row", hit_rate_unweighted, _ema_checks),
    ("calibrate", calibrate_divide_by_T, _ema_checks),
    ("block_mean", mean_divides_by_block_size, _mean_checks),
    ("block_mean", mean_skips_first_token, _mean_checks),
    ("mean_scores", mean_scores_abs, _mean_checks),
    ("fp8_e4m3_decode", fp8_bias_8, _fp8_checks),
    ("fp8_e4m3_decode", fp8_subnormals_flushed, _fp8_checks),
    ("fp8_e4m3_decode", fp8_no_nan, _fp8_checks),
    ("budget_fit", budget_fit_unscaled_x, _budget_checks),
    ("budget_fit", budget_fit_drops_top_power, _budget_checks),
    ("budget_estimates", budget_estimates_never_read_table, _budget_checks),
    ("budget_estimates", budget_estimates_scaled_by_shortest, _budget_checks),
    ("budget_choose", budget_choose_strict, _budget_checks),
    ("budget_choose", budget_choose_smallest, _budget_checks),
    ("budget_blocks", budget_blocks_rounded, _budget_checks),
    ("budget_blocks", budget_blocks_no_slack, _budget_checks),
    ("budget_blocks", budget_blocks_largest_fallback, _budget_checks),
]


@pytest.mark.parametrize("target,mutant,checks", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_pins_catch_planted_mistake(monkeypatch, target, mutant, checks):
    monkeypatch.setattr(orc, target, mutant)
    assert _fails(*checks()), f"no pin noticed the planted mistake {mutant.__name__}"


def test_unmutated_oracle_passes_the_same_checks():
    assert not _fails(*_attention_checks(), *_select_checks(), *_ema_checks(), *_mean_checks(), *_fp8_checks(),
                      *_budget_checks())
