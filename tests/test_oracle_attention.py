"""Pins for the oracle's attention state, merge and repair (CPU only).

What fixes the values here, independent of the oracle's own code:
  * the repair identity: repair(spec(P), M) equals attention over P u M ([paper] §3 design space two,
    §4.3; [blog] Eq. (6));
  * order independence of the merge; M = empty leaves the state untouched; P = empty reduces to plain
    DSA over A ([paper] §3, fall back to recomputation);
  * the dense case against torch's scaled_dot_product_attention in float64 (an independent library);
  * closed forms for one and two tokens and for identical keys;
  * the paged layout decoded against a logical tensor scattered by the test itself.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from _util import oracle_view, random_disjoint_sets, rel_err
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

SMALL = wl.Workload("small", 2, 8, 2, 64, 700, 32, 6, "f32", seed=11, seq_lens=[700, 333])
SMALL_BF16 = wl.scaled(SMALL, name="small_bf16", dtype="bf16", seed=12, head_dim=128)


@pytest.fixture(scope="module", params=[SMALL, SMALL_BF16], ids=lambda w: w.name)
def small(request):
    inp = wl.make_inputs(request.param)
    q, kv = oracle_view(inp)
    return request.param, q[0], kv


def _sets(w, rng, b, n_a, n_b):
    nb = w.blocks_of(b)
    return random_disjoint_sets(rng, nb, n_a, n_b)


def test_paged_layout_decodes_logical_tokens():
    """Scatter a logical K/V into pages with a test-written loop; the oracle's gather must return the
    logical rows (layout only)."""
    rng = np.random.default_rng(0)
    B, Hkv, d, page = 2, 3, 8, 16
    lens = [37, 64]
    max_pages = 4
    perm = rng.permutation(B * max_pages)
    pt = perm.reshape(B, max_pages)
    Klog = rng.standard_normal((B, Hkv, max_pages * page, d))
    Vlog = rng.standard_normal((B, Hkv, max_pages * page, d))
    kc = np.zeros((B * max_pages, Hkv, page, d))
    vc = np.zeros((B * max_pages, Hkv, d, page))
    for b in range(B):
        for h in range(Hkv):
            for t in range(max_pages * page):
                kc[pt[b, t // page], h, t % page, :] = Klog[b, h, t]
                vc[pt[b, t // page], h, :, t % page] = Vlog[b, h, t]
    kv = orc.PagedKV(kc, vc, pt, np.array(lens))
    for b in range(B):
        for h in range(Hkv):
            K, V = orc.gather_kv(kv, b, h, [0, 1, 2], 16)
            n = min(48, lens[b])
            assert np.array_equal(K, Klog[b, h, :n])
            assert np.array_equal(V, Vlog[b, h, :n])
            K, _ = orc.gather_kv(kv, b, h, [2], 32)   # block 2 of 32 starts past both lengths
            assert K.shape[0] == 0


def test_decomposition_identity(small):
    """repair(spec(P), M) == attention over P u M (pin P1)."""
    w, q, kv = small
    rng = np.random.default_rng(1)
    for b in range(w.batch):
        P, M = _sets(w, rng, b, 4, 3)
        for h in range(w.num_q_heads):
            spec = orc.head_state(q, kv, b, h, w.group, P, w.block, w.scale)
            rep = orc.merge(spec, orc.head_state(q, kv, b, h, w.group, M, w.block, w.scale))
            ref = orc.head_state(q, kv, b, h, w.group, sorted(P + M), w.block, w.scale)
            assert abs(rep.m - ref.m) <= 1e-12 * max(1.0, abs(ref.m))
            assert rel_err(rep.l, ref.l) < 1e-12
            assert np.max(np.abs(rep.out - ref.out)) < 1e-12


def test_block_by_block_repair_matches(small):
    """Folding missed blocks one at a time (the blog's per-block application of Eq. (6)) equals
    folding them as one set (pin P2, grouping)."""
    w, q, kv = small
    rng = np.random.default_rng(2)
    b = 0
    P, M = _sets(w, rng, b, 2, 4)
    for h in range(0, w.num_q_heads, 3):
        st = orc.head_state(q, kv, b, h, w.group, P, w.block, w.scale)
        once = orc.merge(st, orc.head_state(q, kv, b, h, w.group, M, w.block, w.scale))
        for blk in M:
            st = orc.merge(st, orc.head_state(q, kv, b, h, w.group, [blk], w.block, w.scale))
        assert rel_err(st.l, once.l) < 1e-12 and abs(st.m - once.m) < 1e-12
        assert np.max(np.abs(st.out - once.out)) < 1e-12


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 10_000), n=st.integers(2, 7))
def test_merge_order_independent(seed, n):
    """Any permutation and grouping of merges gives the same state (pin P2)."""
    rng = np.random.default_rng(seed)
    d = 5
    q = rng.standard_normal(d)
    Ks = [rng.standard_normal((int(rng.integers(0, 4)), d)) * 3 for _ in range(n)]
    Vs = [rng.standard_normal((k.shape[0], d)) for k in Ks]
    states = [orc.attend(q, K, V, 0.7) for K, V in zip(Ks, Vs)]
    whole = orc.attend(q, np.concatenate(Ks), np.concatenate(Vs), 0.7)
    order = rng.permutation(n)
    acc = orc.empty_state(d)
    for i in order:
        acc = orc.merge(acc, states[i])
    # a tree grouping
    tree = states[:]
    while len(tree) > 1:
        tree = [orc.merge(tree[i], tree[i + 1]) if i + 1 < len(tree) else tree[i]
                for i in range(0, len(tree), 2)]
    for s in (acc, tree[0]):
        if whole.m == -math.inf:
            assert s.m == -math.inf and s.l == 0.0
            continue
        assert abs(s.m - whole.m) < 1e-12
        assert rel_err(s.l, whole.l) < 1e-12
        assert np.max(np.abs(s.out - whole.out)) < 1e-12


def test_empty_missed_set_is_identity(small):
    """M = empty leaves (acc, l, m) bit-for-bit unchanged (pin P3)."""
    w, q, kv = small
    P, _ = _sets(w, np.random.default_rng(3), 0, 5, 0)
    st = orc.head_state(q, kv, 0, 1, w.group, P, w.block, w.scale)
    rep = orc.merge(st, orc.head_state(q, kv, 0, 1, w.group, [], w.block, w.scale))
    assert np.array_equal(rep.acc, st.acc) and rep.l == st.l and rep.m == st.m


def test_empty_speculation_is_plain_dsa(small):
    """P = empty: repair from the empty state equals attention over A from scratch (pin P4)."""
    w, q, kv = small
    A, _ = _sets(w, np.random.default_rng(4), 1, 5, 0)
    for h in range(w.num_q_heads):
        rep = orc.merge(orc.empty_state(w.head_dim),
                        orc.head_state(q, kv, 1, h, w.group, A, w.block, w.scale))
        ref = orc.head_state(q, kv, 1, h, w.group, A, w.block, w.scale)
        assert np.array_equal(rep.acc, ref.acc) and rep.l == ref.l and rep.m == ref.m


def test_dense_case_matches_torch_sdpa(small):
    """K >= N and P = empty: the result is ordinary decode attention; checked against torch's
    scaled_dot_product_attention in float64 on the CPU (pin P5)."""
    w, q, kv = small
    for b in range(w.batch):
        nb = w.blocks_of(b)
        L = w.lengths[b]
        for h in range(w.num_q_heads):
            st = orc.merge(orc.empty_state(w.head_dim),
                           orc.head_state(q, kv, b, h, w.group, list(range(nb)), w.block, w.scale))
            # logical K/V of the whole sequence, read straight from the pages by the test
            toks = np.arange(L)
            pages = kv.page_table[b, toks // 16]
            K = kv.k[pages, h // w.group, toks % 16, :]
            V = kv.v[pages, h // w.group, :, toks % 16]
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h][None, None, None, :]),
                torch.from_numpy(np.ascontiguousarray(K)[None, None]),
                torch.from_numpy(np.ascontiguousarray(V)[None, None]), scale=w.scale)
            assert np.max(np.abs(st.out - ref.numpy()[0, 0, 0])) < 1e-12


def test_closed_forms():
    """One token: O = v, l = 1, m = s.  Two tokens: softmax-weighted mean.  Identical keys in a
    block: O = mean(v), l = n (pin P6)."""
    d = 4
    q = np.array([0.5, -1.0, 2.0, 0.25])
    k = np.array([[1.0, 2.0, -0.5, 4.0]])
    v = np.array([[3.0, -2.0, 1.0, 0.5]])
    st = orc.attend(q, k, v, 0.125)
    s = 0.125 * (0.5 * 1.0 + (-1.0) * 2.0 + 2.0 * (-0.5) + 0.25 * 4.0)
    assert st.l == 1.0 and abs(st.m - s) < 1e-15 and np.allclose(st.out, v[0], atol=0, rtol=1e-15)
    k2 = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 1.0, 0.0]])
    v2 = np.array([[1.0, 2.0, 3.0, 4.0], [-1.0, 0.0, 1.0, 8.0]])
    st = orc.attend(q, k2, v2, 1.0)
    s1, s2 = 0.5, 2.0
    w1, w2 = math.exp(s1 - s2), 1.0
    expect = (w1 * v2[0] + w2 * v2[1]) / (w1 + w2)
    assert abs(st.m - 2.0) < 1e-15 and abs(st.l - (w1 + w2)) < 1e-15
    assert np.max(np.abs(st.out - expect)) < 1e-15
    kk = np.tile(np.array([[0.3, -0.2, 0.1, 0.9]]), (6, 1))
    vv = np.random.default_rng(0).standard_normal((6, d))
    st = orc.attend(q, kk, vv, 0.5)
    assert abs(st.l - 6.0) < 1e-15 and np.max(np.abs(st.out - vv.mean(axis=0))) < 1e-15


def test_empty_state_conventions():
    st = orc.attend(np.ones(3), np.zeros((0, 3)), np.zeros((0, 3)), 1.0)
    assert st.l == 0.0 and st.m == -math.inf and np.array_equal(st.acc, np.zeros(3))
    both = orc.merge(st, st)
    assert both.l == 0.0 and both.m == -math.inf and np.array_equal(both.out, np.zeros(3))
