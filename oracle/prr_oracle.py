"""CPU oracle for the PRR decode hot path.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's cpu-baseline leg may import this module.
The product path (the HIP library and its Python binding) never calls it, and it imports nothing from
the product: it shares no code with the GPU path.  Everything here is plain NumPy in float64, written
so that it can be checked against the pages by eye.

Citations:
  [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM
          Decoding" (full paper text)
  [blog]  "PRR: Predict, Reuse, and Repair - Accelerating Dynamic Sparse Attention for Long-Context
          LLM Decoding" (xllm-io paper review; carries the equation numbers (1)-(6))

Readings taken where the pages are silent (each is also listed in the design notes):
  * softmax scale: the caller's fp32 `scale` (1/sqrt(d) by default), promoted to float64;
  * kv head of query head h is h // G (contiguous grouping);
  * the attention state is (acc, l, m) with acc unnormalised: O = acc / l; m in natural-log units;
  * Quest sums run sequentially over channels 0..d-1 from +0.0 with separate multiply and add;
    the representative query sums the G heads in order g = 0..G-1 from +0.0, then divides by G;
  * top-K ties go to the smaller block index; K larger than the number of blocks selects all;
  * EMA: (1 - alpha) and (1 - beta) are formed as 1.0 - x in float64; a block born at step tau gets
    level = IS^tau, trend = 0;
  * calibration: rows phi = 1 .. T_p-1 are scored (row 0 only initialises), H is their mean, the
    argmax is the first maximum in grid order (alpha-major, then beta, then gamma).

Parity status: every function below is pinned by tests/test_oracle_*.py against closed forms,
invariants, brute force or an independent library routine.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Iterable, List, Sequence

import numpy as np

# --------------------------------------------------------------------------------------------------
# Storage decoding (layout only)
# --------------------------------------------------------------------------------------------------


def fp8_e4m3_decode(codes) -> np.ndarray:
    """Values of 8-bit E4M3 floating-point codes (the OCP 8-bit format in its FN variant: no
    infinities): bit 7 the sign, bits 6-3 the exponent field E (bias 7), bits 2-0 the mantissa field M.
    E = 0 holds the subnormals M * 2^-9 (and the zeros); otherwise the value is (1 + M/8) * 2^(E - 7);
    E = 15 with M = 7 is NaN, so the largest finite magnitude is 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def upcast(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored elements: raw bf16 bit patterns (uint16), fp32, or for an fp8
    cache its E4M3 codes (uint8); an fp8 cache keeps queries and min/max metadata in bf16, so uint16
    arrays under "fp8" are bf16 bit patterns."""
    if dtype == "fp8":
        a = np.asarray(arr)
        return upcast(a, "bf16") if a.dtype == np.uint16 else fp8_e4m3_decode(a)
    if dtype == "bf16":
        a = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << 16
        return a.view(np.float32).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


@dataclass
class PagedKV:
    """Host copy of the paged cache.

    k [num_pages][Hkv][page][d] (token-major tiles), v [num_pages][Hkv][d][page] (channel-major tiles),
    page_table [B][max_pages], seq_len [B].  Values are already float64."""

    k: np.ndarray
    v: np.ndarray
    page_table: np.ndarray
    seq_len: np.ndarray

    @property
    def page(self) -> int:
        return self.k.shape[2]

    @property
    def head_dim(self) -> int:
        return self.k.shape[3]


def make_paged_kv(k_bits, v_bits, page_table, seq_len, dtype: str) -> PagedKV:
    return PagedKV(upcast(k_bits, dtype), upcast(v_bits, dtype),
                   np.asarray(page_table, dtype=np.int64), np.asarray(seq_len, dtype=np.int64))


def num_blocks(kv: PagedKV, b: int, block: int) -> int:
    """Blocks of sequence b: ceil(seq_len / block); a partial last block is still a block."""
    return -(-int(kv.seq_len[b]) // block)


def block_token_ids(kv: PagedKV, b: int, blocks: Iterable[int], block: int) -> List[int]:
    """Logical token positions covered by the given blocks of sequence b (valid tokens only)."""
    L = int(kv.seq_len[b])
    out = []
    for p in blocks:
        lo = int(p) * block
        out.extend(range(lo, min(lo + block, L)))
    return out


def gather_kv(kv: PagedKV, b: int, kvh: int, blocks: Iterable[int], block: int):
    """Keys [n][d] and values [n][d] (float64) of the valid tokens of `blocks` in sequence b."""
    toks = block_token_ids(kv, b, blocks, block)
    if not toks:
        d = kv.head_dim
        return np.zeros((0, d)), np.zeros((0, d))
    toks = np.asarray(toks, dtype=np.int64)
    pages = kv.page_table[b, toks // kv.page]
    offs = toks % kv.page
    return kv.k[pages, kvh, offs, :], kv.v[pages, kvh, :, offs]


# --------------------------------------------------------------------------------------------------
# Attention state over a block set, and the repair merge
# --------------------------------------------------------------------------------------------------


@dataclass
class State:
    """Partial attention state of one query head: acc = sum_j e^{s_j - m} v_j, l = sum_j e^{s_j - m},
    m = max_j s_j.  The empty state is (0, 0, -inf)."""

    acc: np.ndarray
    l: float
    m: float

    @property
    def out(self) -> np.ndarray:
        return self.acc / self.l if self.l > 0 else np.zeros_like(self.acc)


def empty_state(d: int) -> State:
    return State(np.zeros(d), 0.0, -math.inf)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> State:
    """Softmax attention of one query over a token set, kept as an unnormalised state.

    The speculative kernel's extra outputs are the softmax denominator and running maximum
    ([paper] §4.3, instrumented speculative kernel; [blog] Eq. (6) commentary)."""
    if K.shape[0] == 0:
        return empty_state(q.shape[0])
    s = (K @ q) * float(scale)
    m = float(np.max(s))
    e = np.exp(s - m)
    return State(e @ V, float(np.sum(e)), m)


def merge(a: State, b: State) -> State:
    """Fold state b into state a with the online-softmax recurrence ([paper] §4.3 repair recurrence;
    [blog] Eq. (6)), written for unnormalised accumulators:
      m' = max(m_a, m_b);  l' = e^{m_a-m'} l_a + e^{m_b-m'} l_b;  acc' = e^{m_a-m'} acc_a + e^{m_b-m'} acc_b.
    With O = acc/l this is exactly Eq. (6).  A side with m = -inf (no tokens) contributes nothing."""
    m = max(a.m, b.m)
    if m == -math.inf:
        return State(a.acc + b.acc, 0.0, -math.inf)
    fa = 0.0 if a.m == -math.inf else math.exp(a.m - m)
    fb = 0.0 if b.m == -math.inf else math.exp(b.m - m)
    return State(fa * a.acc + fb * b.acc, fa * a.l + fb * b.l, m)


def head_state(q_all: np.ndarray, kv: PagedKV, b: int, h: int, G: int, blocks: Sequence[int],
               block: int, scale: float) -> State:
    """Attention state of query head h of sequence b over `blocks` (kv head = h // G)."""
    K, V = gather_kv(kv, b, h // G, blocks, block)
    return attend(q_all[b, h], K, V, scale)


def spec_states(q_all: np.ndarray, kv: PagedKV, block: int, P: Sequence[Sequence[Sequence[int]]],
                scale: float, heads: Iterable = None):
    """Speculative attention over the predicted set P[b][kvh] for every query head
    ([paper] §3 and §4.3; P is shared by the G query heads of a kv head, [paper] A.1).
    Returns {(b, h): State}."""
    B, Hq, _ = q_all.shape
    Hkv = len(P[0])
    G = Hq // Hkv
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    return {(b, h): head_state(q_all, kv, b, h, G, P[b][h // G], block, scale) for b, h in heads}


def repair_states(states: dict, q_all: np.ndarray, kv: PagedKV, block: int,
                  M: Sequence[Sequence[Sequence[int]]], scale: float) -> dict:
    """Incremental repair: fold the missed blocks M = A \\ P into the speculative states
    ([paper] §3 design space two, §4.3; [blog] Eq. (6)).  The missed blocks are attended as one
    token set and merged once; folding them block by block gives the same value up to rounding."""
    Hq = q_all.shape[1]
    Hkv = len(M[0])
    G = Hq // Hkv
    out = {}
    for (b, h), st in states.items():
        out[(b, h)] = merge(st, head_state(q_all, kv, b, h, G, M[b][h // G], block, scale))
    return out


# --------------------------------------------------------------------------------------------------
# Quest selection, GQA-extended
# --------------------------------------------------------------------------------------------------


def block_minmax(kv: PagedKV, b: int, kvh: int, p: int, block: int):
    """Channel-wise min and max keys of block p of sequence b over its valid tokens
    ([paper] A.1, page metadata m_p, M_p kept per KV head)."""
    K, _ = gather_kv(kv, b, kvh, [p], block)
    return K.min(axis=0), K.max(axis=0)


def build_meta(kv: PagedKV, block: int, Hkv: int) -> list:
    """[b][kvh] -> (mn [N_b][d], mx [N_b][d]) for every block of every sequence."""
    out = []
    for b in range(kv.seq_len.shape[0]):
        row = []
        for h in range(Hkv):
            nb = num_blocks(kv, b, block)
            mn = np.empty((nb, kv.head_dim))
            mx = np.empty((nb, kv.head_dim))
            for p in range(nb):
                mn[p], mx[p] = block_minmax(kv, b, h, p, block)
            row.append((mn, mx))
        out.append(row)
    return out


def block_mean(kv: PagedKV, b: int, kvh: int, p: int, block: int) -> np.ndarray:
    """Channel-wise mean key of block p over its valid tokens: the block compressed to one representative
    ([paper] §2.1: selection compresses each block, e.g. by its mean).  The tokens are summed one after
    another from +0.0 in float64, the sum is divided by their count, and the mean is rounded once to
    float32 (the stored summary)."""
    K, _ = gather_kv(kv, b, kvh, [p], block)
    acc = np.zeros(K.shape[1])
    for t in range(K.shape[0]):
        acc = acc + K[t]
    return (acc / K.shape[0]).astype(np.float32).astype(np.float64)


def build_mean_meta(kv: PagedKV, block: int, Hkv: int) -> list:
    """[b][kvh] -> mean [N_b][d] for every block of every sequence."""
    out = []
    for b in range(kv.seq_len.shape[0]):
        row = []
        for h in range(Hkv):
            nb = num_blocks(kv, b, block)
            mean = np.empty((nb, kv.head_dim))
            for p in range(nb):
                mean[p] = block_mean(kv, b, h, p, block)
            row.append(mean)
        out.append(row)
    return out


def mean_scores(qbar: np.ndarray, mean: np.ndarray) -> np.ndarray:
    """Mean-pooled criticality s_p = sum_i Qbar_i mean_{p,i} for every block p, channels added one after
    another from +0.0 with a separate multiply and add.  mean: [N][d]."""
    s = np.zeros(mean.shape[0])
    for i in range(mean.shape[1]):
        s = s + qbar[i] * mean[:, i]
    return s


def select_mean(q_all: np.ndarray, mean_meta: list, G: int, k: int, P=None):
    """Selection with mean-pooled scores for every (b, kvh): scores, A = top-k, M = A \\ P."""
    scores, A, M = [], [], []
    for b in range(len(mean_meta)):
        srow, arow, mrow = [], [], []
        for h in range(len(mean_meta[0])):
            s = mean_scores(representative_query(q_all, b, h, G), mean_meta[b][h])
            a = topk_blocks(s, k)
            srow.append(s)
            arow.append(a)
            mrow.append(set_minus(a, P[b][h]) if P is not None else None)
        scores.append(srow)
        A.append(arow)
        M.append(mrow)
    return scores, A, M


def representative_query(q_all: np.ndarray, b: int, kvh: int, G: int) -> np.ndarray:
    """Q_bar = (1/G) sum_g Q_g over the G query heads sharing kv head kvh ([paper] A.1)."""
    acc = np.zeros(q_all.shape[2])
    for g in range(G):
        acc = acc + q_all[b, kvh * G + g]
    return acc / G


def quest_scores(qbar: np.ndarray, mn: np.ndarray, mx: np.ndarray) -> np.ndarray:
    """Criticality s_p = sum_i max(Qbar_i m_{p,i}, Qbar_i M_{p,i}) for every block p ([paper] A.1).
    mn, mx: [N][d].  Channels are added one after another starting from +0.0."""
    s = np.zeros(mn.shape[0])
    for i in range(mn.shape[1]):
        s = s + np.maximum(qbar[i] * mn[:, i], qbar[i] * mx[:, i])
    return s


def topk_blocks(scores: np.ndarray, k: int) -> np.ndarray:
    """The k highest-scoring blocks, ties to the smaller index, returned in ascending block order
    ([paper] §1 and §2.1, top-K selection; [paper] A.1, top-K pages per KV head)."""
    n = scores.shape[0]
    k = max(0, min(int(k), n))
    order = np.lexsort((np.arange(n), -scores))   # primary: score descending; then index ascending
    return np.sort(order[:k]).astype(np.int64)


def set_minus(a: Sequence[int], b: Sequence[int]) -> np.ndarray:
    """Ascending a \\ b ([paper] §3: missed blocks M = A \\ P, wasted blocks N = P \\ A)."""
    return np.setdiff1d(np.asarray(a, dtype=np.int64), np.asarray(b, dtype=np.int64))


def select(q_all: np.ndarray, meta: list, G: int, k: int, P=None):
    """Quest selection for every (b, kvh): scores, A = top-k, and M = A \\ P when P is given."""
    B = len(meta)
    Hkv = len(meta[0])
    scores, A, M = [], [], []
    for b in range(B):
        srow, arow, mrow = [], [], []
        for h in range(Hkv):
            mn, mx = meta[b][h]
            s = quest_scores(representative_query(q_all, b, h, G), mn, mx)
            a = topk_blocks(s, k)
            srow.append(s)
            arow.append(a)
            mrow.append(set_minus(a, P[b][h]) if P is not None else None)
        scores.append(srow)
        A.append(arow)
        M.append(mrow)
    return scores, A, M


# --------------------------------------------------------------------------------------------------
# EMA level/trend predictor
# --------------------------------------------------------------------------------------------------


def ema_update(level: np.ndarray, trend: np.ndarray, IS: np.ndarray, alpha: float, beta: float):
    """One update with the observed scores ([paper] §4.1; [blog] Eq. (3)):
    v^t = beta (IS^t - l^{t-1}) + (1 - beta) v^{t-1};  l^t = alpha IS^t + (1 - alpha) l^{t-1}.
    Both right-hand sides use the previous level."""
    one_a = 1.0 - alpha
    one_b = 1.0 - beta
    t = IS - level
    new_trend = beta * t + one_b * trend
    new_level = alpha * IS + one_a * level
    return new_level, new_trend


def ema_predict(level: np.ndarray, trend: np.ndarray, gamma: float) -> np.ndarray:
    """Predicted scores ([paper] §4.1; [blog] Eq. (2)): IS_hat^t = l^{t-1} + gamma v^{t-1}."""
    return level + gamma * trend


def predict_step(level: np.ndarray, trend: np.ndarray, live: int, IS: np.ndarray, alpha: float,
                 beta: float, gamma: float, budget: int):
    """Advance one (b, kvh) predictor by one decode step and propose the next speculative set.

    Blocks [0, live) carry state and get the Eq. (3) update; blocks [live, len(IS)) enter now and
    start at level = IS, trend = 0 ([paper] §4.1, state and initialisation).  The next set P is the
    `budget` blocks with the highest Eq. (2) prediction (ties to the smaller index).
    Returns (level, trend, live', P_next)."""
    n = IS.shape[0]
    lv = np.empty(n)
    tr = np.empty(n)
    lv[:live], tr[:live] = ema_update(level[:live], trend[:live], IS[:live], alpha, beta)
    lv[live:] = IS[live:]
    tr[live:] = 0.0
    pred = ema_predict(lv, tr, gamma)
    return lv, tr, n, topk_blocks(pred, budget)


# --------------------------------------------------------------------------------------------------
# Online predictor calibration
# --------------------------------------------------------------------------------------------------


def calibration_grid() -> np.ndarray:
    """alpha in [0.2, 0.8] step 0.2, beta in [0.1, 0.5] step 0.1, gamma in [0, 0.75] step 0.25,
    endpoints included: 4 x 5 x 4 = 80 candidates ([paper] §4.2; [blog] search procedure).
    Values are the decimal literals, alpha-major."""
    alphas = [0.2, 0.4, 0.6, 0.8]
    betas = [0.1, 0.2, 0.3, 0.4, 0.5]
    gammas = [0.0, 0.25, 0.5, 0.75]
    return np.array([[a, b, g] for a in alphas for b in betas for g in gammas], dtype=np.float64)


def hit_rate_row(IS_row: np.ndarray, P: np.ndarray, A: np.ndarray) -> float:
    """Score-weighted hit rate of one row: sum_{b in P n A} IS_b / sum_{b in A} IS_b
    ([paper] §4.2; [blog] Eq. (4), summand)."""
    hit = np.intersect1d(P, A)
    den = 0.0
    for b in np.sort(A):
        den += IS_row[b]
    num = 0.0
    for b in np.sort(hit):
        num += IS_row[b]
    return num / den if den != 0.0 else 0.0


def calibrate(IS: np.ndarray, k: int, grid: np.ndarray = None):
    """Grid search for the predictor parameters ([paper] §4.2; [blog] Eqs. (4)-(5)).

    For every theta the EMA runs over the prefill rows: row 0 initialises (level = IS_0, trend = 0);
    for each later row phi the prediction picks P_phi(theta) = top-k, A_phi = top-k of the true row,
    h_phi is the score-weighted hit rate, then the state is updated with row phi.
    H(theta) is the mean of h_phi over phi = 1 .. T_p-1; theta* is the first argmax.
    Returns (H [n], best index)."""
    if grid is None:
        grid = calibration_grid()
    IS = np.asarray(IS, dtype=np.float64)
    T = IS.shape[0]
    A = [topk_blocks(IS[phi], k) for phi in range(T)]
    H = np.zeros(grid.shape[0])
    for j, (alpha, beta, gamma) in enumerate(grid):
        level = IS[0].copy()
        trend = np.zeros(IS.shape[1])
        total = 0.0
        for phi in range(1, T):
            P = topk_blocks(ema_predict(level, trend, gamma), k)
            total += hit_rate_row(IS[phi], P, A[phi])
            level, trend = ema_update(level, trend, IS[phi], alpha, beta)
        H[j] = total / (T - 1) if T > 1 else 0.0
    best = int(np.argmax(H))   # first maximum in grid order
    return H, best


# --------------------------------------------------------------------------------------------------
# Critical-path-aware speculation budget ([paper] §4.4, A.6; [blog] Eq. (1))
# --------------------------------------------------------------------------------------------------


def budget_fit(ctx, t_select, deltas, t_spec, degree: int) -> np.ndarray:
    """Polynomial regression of the profiled latencies over context length ([paper] A.6: lengths outside
    the profiled grid are estimated by polynomial regression).  Reading (the pages name no degree, basis
    or fitting criterion): ordinary least squares of `degree` in x = T / max(ctx), one polynomial for
    the selection latency and one per budget ratio for the speculative latency (t_spec[j][i] at
    deltas[j], ctx[i]).  Returns coef [1 + len(deltas)][degree + 1], coef[r][k] multiplying x^k, row 0
    selection.  The least-squares solve is numpy.linalg.lstsq."""
    ctx = np.asarray(ctx, dtype=np.float64)
    x = ctx / ctx[-1]
    V = np.vander(x, degree + 1, increasing=True)
    rows = [np.asarray(t_select, dtype=np.float64)] + [np.asarray(r, dtype=np.float64) for r in t_spec]
    return np.array([np.linalg.lstsq(V, y, rcond=None)[0] for y in rows])


def budget_estimates(ctx, t_select, t_spec, coef: np.ndarray, context: float) -> np.ndarray:
    """Latency estimates at `context` tokens ([paper] §4.4: the profiles are a table indexed by context
    length; A.6: regression for lengths outside it): the profiled row itself at a profiled length, else
    sum_k coef[r][k] x^k with x = context / max(ctx).  Returns [est_select, est_spec(delta_0), ...]."""
    ctx = [float(c) for c in ctx]
    if float(context) in ctx:
        i = ctx.index(float(context))
        return np.array([float(t_select[i])] + [float(r[i]) for r in t_spec])
    x = float(context) / ctx[-1]
    return np.array([sum(c * x ** k for k, c in enumerate(row)) for row in coef])


def budget_blocks(deltas, choice: int, topk: int) -> int:
    """|P| in blocks for the chosen ratio ([blog] Eq. (1): |P| <= delta |A|, with |A| = topk).  Reading: the
    largest set the constraint admits, floor(delta topk) (the product in float64 with a relative slack of
    1e-9, so that a product that rounds just below an integer still reaches it); when no ratio fits
    (choice -1), the smallest profiled ratio (speculating over fewer blocks leaves more to repair, which
    is on the critical path too)."""
    d = float(deltas[choice if choice >= 0 else 0])
    x = d * float(topk)
    return int(np.floor(x + 1e-9 * max(1.0, x)))


def budget_choose(ctx, t_select, deltas, t_spec, coef: np.ndarray, context: float):
    """The largest profiled budget ratio whose speculative latency is at most the selection latency at
    `context` tokens ([paper] §4.4: speculation must not outlast selection, else it extends the critical
    path).  Reading: 'fits' is est_spec <= est_select; -1 when no ratio fits.  Returns (index, estimates)."""
    est = budget_estimates(ctx, t_select, t_spec, coef, context)
    fits = [j for j in range(len(deltas)) if est[1 + j] <= est[0]]
    return (max(fits) if fits else -1), est
