"""Pins for the oracle's mean-pooled block scoring (CPU only).

Selection compresses each block to one representative and scores it against the query ([paper] §2.1:
"e.g., mean"); the mean-pooled variant keeps each block's channel-wise mean key (float64 sum in token
order, divided by the token count, rounded once to float32).  Independent facts used:
  * a block whose valid tokens share one key has that key as its mean, full or partial (a divisor other
    than the valid-token count fails here);
  * the mean lies between the block's min and max keys, channel by channel, so the mean-pooled score is
    bounded by the Quest score bit for bit (every step of both float64 sums is monotone);
  * for one-token blocks the score is q_bar . k, the same as numpy's dot product to rounding;
  * the mean agrees with numpy's mean over the block's tokens to float32 rounding.
"""
import numpy as np
import pytest

from _util import oracle_view
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

W = wl.Workload("mean", 2, 8, 2, 64, 900, 16, 7, "bf16", seed=23, seq_lens=[900, 517])


@pytest.fixture(scope="module")
def fx():
    inp = wl.make_inputs(W)
    q, kv = oracle_view(inp)
    return q[0], kv, orc.build_meta(kv, W.block, W.num_kv_heads), orc.build_mean_meta(kv, W.block, W.num_kv_heads)


def test_mean_matches_numpy_mean(fx):
    q, kv, _, mean = fx
    for b in range(W.batch):
        for h in range(W.num_kv_heads):
            for p in range(mean[b][h].shape[0]):
                K, _ = orc.gather_kv(kv, b, h, [p], W.block)
                ref = np.mean(K, axis=0)
                assert np.all(np.abs(mean[b][h][p] - ref) <= 2.0 ** -23 * np.maximum(np.abs(ref), 2.0 ** -126)
                              + 1e-12), (b, h, p)
                assert np.array_equal(mean[b][h][p], mean[b][h][p].astype(np.float32)), "float32 values"


def test_mean_score_bounded_by_quest_score(fx):
    q, kv, meta, mean = fx
    for b in range(W.batch):
        for h in range(W.num_kv_heads):
            mn, mx = meta[b][h]
            assert np.all(mean[b][h] >= mn) and np.all(mean[b][h] <= mx)
            qbar = orc.representative_query(q, b, h, W.group)
            assert np.all(orc.mean_scores(qbar, mean[b][h]) <= orc.quest_scores(qbar, mn, mx))


def test_identical_keys_and_partial_blocks():
    """Every token of a block carries the same key (blocks of 16, the last one partial): the mean is that
    key exactly and the score is the query-key product."""
    w = wl.Workload("mean_const", 1, 4, 1, 64, 16 * 9 + 5, 16, 4, "bf16", seed=24, shuffle_pages=False)
    inp = wl.make_inputs(w)
    # key of block p = the block's first token, copied over its other tokens
    for p in range(w.blocks_of(0)):
        inp.k_cache[p, :, :, :] = inp.k_cache[p, :, 0:1, :]
    q, kv = oracle_view(inp)
    mean = orc.build_mean_meta(kv, w.block, 1)[0][0]
    for p in range(mean.shape[0]):
        assert np.array_equal(mean[p], kv.k[p, 0, 0]), p
    qbar = orc.representative_query(q[0], 0, 0, w.group)
    s = orc.mean_scores(qbar, mean)
    assert np.allclose(s, mean @ qbar, rtol=1e-12, atol=1e-12)


def test_single_token_blocks_score_is_dot_product():
    w = wl.Workload("mean_one", 1, 8, 2, 64, 16 * 6, 16, 4, "bf16", seed=25, shuffle_pages=False)
    inp = wl.make_inputs(w)
    q, kv = oracle_view(inp)
    for h in range(w.num_kv_heads):
        qbar = orc.representative_query(q[0], 0, h, w.group)
        # one-token blocks: a 1-token cache per block is the prefix of each 16-token block
        one = orc.make_paged_kv(wl.to_numpy_bits(inp.k_cache), wl.to_numpy_bits(inp.v_cache),
                                np.arange(inp.k_cache.shape[0]).reshape(1, -1), np.array([1]), w.dtype)
        mean = orc.build_mean_meta(one, 16, w.num_kv_heads)[0][h]
        assert np.allclose(orc.mean_scores(qbar, mean), kv.k[0, h, 0] @ qbar, rtol=1e-12, atol=1e-12)


def test_select_mean_is_topk_of_mean_scores(fx):
    q, kv, _, mean = fx
    P = [[[0, 3, 5], [1]], [[2, 4], []]]
    scores, A, M = orc.select_mean(q, mean, W.group, W.topk, P)
    for b in range(W.batch):
        for h in range(W.num_kv_heads):
            qbar = orc.representative_query(q, b, h, W.group)
            s = orc.mean_scores(qbar, mean[b][h])
            assert np.array_equal(scores[b][h], s)
            assert np.array_equal(A[b][h], orc.topk_blocks(s, W.topk))
            assert np.array_equal(M[b][h], orc.set_minus(A[b][h], P[b][h]))
