"""Pins for the oracle's Quest selection and top-K (CPU only).

Independent facts used ([paper] A.1 extends Quest to GQA with a representative query and channel-wise
min/max page metadata; [paper] §1 and §2.1 top-K block selection):
  * the Quest score is an upper bound of q_bar . k over the block's tokens, with equality when a block
    holds one token (min = max);
  * with G = 1 the representative query is the head's own query (original per-head Quest);
  * the representative query equals numpy's mean over the group;
  * min/max metadata equals a brute-force scan of the block's tokens;
  * top-K equals heapq.nlargest on (score, -index) tuples, ties included;
  * planted heavy blocks are always selected.
"""
import heapq

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from _util import oracle_view
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

W = wl.Workload("sel", 2, 8, 2, 64, 900, 16, 7, "bf16", seed=21, seq_lens=[900, 517])


@pytest.fixture(scope="module")
def sel():
    inp = wl.make_inputs(W)
    q, kv = oracle_view(inp)
    return q[0], kv, orc.build_meta(kv, W.block, W.num_kv_heads)


def test_meta_is_brute_force_minmax(sel):
    q, kv, meta = sel
    for b in range(W.batch):
        L = W.lengths[b]
        for h in range(W.num_kv_heads):
            mn, mx = meta[b][h]
            assert mn.shape[0] == -(-L // W.block)
            for p in range(mn.shape[0]):
                rows = []
                for t in range(p * W.block, min(L, (p + 1) * W.block)):
                    rows.append(kv.k[kv.page_table[b, t // 16], h, t % 16])
                rows = np.array(rows)
                assert np.array_equal(mn[p], rows.min(axis=0))
                assert np.array_equal(mx[p], rows.max(axis=0))


def test_quest_score_is_upper_bound(sel):
    """s_p >= max_{t in p} q_bar . k_t for every block (why the criterion is safe)."""
    q, kv, meta = sel
    for b in range(W.batch):
        for h in range(W.num_kv_heads):
            qbar = orc.representative_query(q, b, h, W.group)
            mn, mx = meta[b][h]
            s = orc.quest_scores(qbar, mn, mx)
            for p in range(s.shape[0]):
                K, _ = orc.gather_kv(kv, b, h, [p], W.block)
                assert s[p] >= np.max(K @ qbar) - 1e-9 * (1 + abs(s[p]))


def test_single_token_blocks_give_exact_dot():
    """min = max (one token per block): the score is q_bar . k."""
    rng = np.random.default_rng(5)
    qbar = rng.standard_normal(32)
    k = rng.standard_normal((50, 32))
    s = orc.quest_scores(qbar, k, k)
    assert np.max(np.abs(s - k @ qbar)) < 1e-12


def test_representative_query_is_group_mean(sel):
    q, _, _ = sel
    for b in range(W.batch):
        for h in range(W.num_kv_heads):
            ref = np.mean(q[b, h * W.group:(h + 1) * W.group], axis=0)
            assert np.max(np.abs(orc.representative_query(q, b, h, W.group) - ref)) < 1e-15
    # G = 1 is the original per-head criterion
    assert np.array_equal(orc.representative_query(q, 0, 3, 1), q[0, 3])


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 100_000), n=st.integers(1, 40), k=st.integers(0, 45),
       levels=st.integers(1, 6))
def test_topk_matches_heapq_with_ties(seed, n, k, levels):
    """Brute force: heapq.nlargest over (score, -index); integer scores force ties."""
    rng = np.random.default_rng(seed)
    s = rng.integers(0, levels, size=n).astype(np.float64)
    got = orc.topk_blocks(s, k)
    ref = sorted(-negj for _, negj in heapq.nlargest(min(k, n), [(s[j], -j) for j in range(n)]))
    assert list(got) == ref
    assert list(got) == sorted(got) and len(set(got)) == len(got)


def test_topk_edge_cases():
    s = np.array([3.0, 1.0, 2.0])
    assert list(orc.topk_blocks(s, 0)) == []
    assert list(orc.topk_blocks(s, 10)) == [0, 1, 2]
    assert list(orc.topk_blocks(np.array([-1.0, -1.0, -2.0]), 1)) == [0]
    assert list(orc.set_minus([1, 4, 7, 9], [9, 2, 4])) == [1, 7]
    assert list(orc.set_minus([], [1])) == []


def test_planted_blocks_are_selected():
    """Keys of planted blocks carry +c * q_hat, so every planted block lands in A (pin P9)."""
    w = wl.scaled(wl.C2, name="c2_small", context=4096, topk=48, planted=12, spec_hit=-1)
    inp = wl.make_inputs(w)
    q, kv = oracle_view(inp)
    meta = orc.build_meta(kv, w.block, w.num_kv_heads)
    _, A, _ = orc.select(q[0], meta, w.group, w.topk)
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            assert set(inp.planted[b, h].tolist()) <= set(A[b][h].tolist())
