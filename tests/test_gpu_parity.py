"""GPU parity: libprr.so through the C ABI against the CPU oracle on the same seeded inputs.

Block indices, sets, scores, metadata and EMA state must match bit for bit; the attention state must
match within O 5e-3 (max abs), l 1e-4 (relative), m 1e-4 (relative).
"""
import math

import numpy as np
import pytest
import torch

from _gpu import (assert_heads, assert_state, device_kv, require_gpu, sets_to_device, unit_meta,
                  unit_view)
from _util import oracle_view
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


def _meta_bits(meta: torch.Tensor, w: wl.Workload):
    # columns past each sequence's block count are never written (arbitrary bits)
    with np.errstate(invalid="ignore"):
        return orc.upcast(wl.to_numpy_bits(meta), w.dtype)


# --------------------------------------------------------------------------------------------------
# Tiny configuration end to end
# --------------------------------------------------------------------------------------------------


def test_tiny_end_to_end():
    w = wl.C1
    inp = wl.make_inputs(w, "cuda")
    q, kv = oracle_view(inp)
    q = q[0]
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    ometa = orc.build_meta(kv, w.block, w.num_kv_heads)
    gm = _meta_bits(meta, w)
    nb = w.blocks_of(0)
    assert np.array_equal(gm[0, 0, :, 0, :nb].T, ometa[0][0][0])
    assert np.array_equal(gm[0, 0, :, 1, :nb].T, ometa[0][0][1])

    scores, A, _ = bd.select(inp.q[0], dkv, meta, w.block, w.topk)
    oscores, oA, _ = orc.select(q, ometa, w.group, w.topk)
    assert np.array_equal(scores[0, 0, :nb].cpu().numpy(), oscores[0][0])
    assert A.lists()[0][0] == list(oA[0][0])

    P = [[wl.make_spec_set(w, oA[0][0], nb, w.spec_hit, w.spec_miss)]]
    Pd = sets_to_device(P, w.topk)
    _, A2, M = bd.select(inp.q[0], dkv, meta, w.block, w.topk, P=Pd)
    oM = orc.set_minus(oA[0][0], P[0][0])
    assert A2.lists()[0][0] == list(oA[0][0])
    assert M.lists()[0][0] == list(oM) and len(oM) == 3

    state = bd.spec_attn(inp.q[0], dkv, w.block, Pd, w.scale)
    spec_ref = orc.spec_states(q, kv, w.block, P, w.scale)
    assert_heads(state, spec_ref, "spec")
    out = torch.empty_like(state.acc)
    bd.repair(inp.q[0], dkv, w.block, M, w.scale, state, out=out)
    union = [[sorted(set(P[0][0]) | set(oM))]]
    ref = orc.spec_states(q, kv, w.block, union, w.scale)
    assert_heads(state, ref, "repair")
    for h in range(w.num_q_heads):
        assert np.max(np.abs(out[0, h].double().cpu().numpy() - ref[(0, h)].out)) <= 5e-3


# --------------------------------------------------------------------------------------------------
# Small shapes: head dims, group sizes, block sizes, ragged lengths, empty sets
# --------------------------------------------------------------------------------------------------

CASES = [
    # name, B, Hq, Hkv, d, block, lens, dtype
    ("bf16_d128_g4_s16", 2, 8, 2, 128, 16, [1000, 611], "bf16"),
    ("bf16_d128_g4_s64", 2, 8, 2, 128, 64, [2048, 1500], "bf16"),
    ("bf16_d64_g8_s32", 1, 16, 2, 64, 32, [1777], "bf16"),
    ("bf16_d128_g16_s32", 1, 16, 1, 128, 32, [900], "bf16"),
    ("bf16_d128_g1_s16", 1, 4, 4, 128, 16, [333], "bf16"),
    ("bf16_d128_g2_s48", 2, 4, 2, 128, 48, [960, 97], "bf16"),
    ("bf16_d128_g4_s128", 2, 8, 2, 128, 128, [6144, 4999], "bf16"),
    ("bf16_d128_g4_s256", 1, 8, 2, 128, 256, [8192 - 77], "bf16"),
    ("fp8_d128_g4_s256", 2, 8, 2, 128, 256, [7000, 8192], "fp8"),
    ("fp8_d128_g4_s16", 2, 8, 2, 128, 16, [1000, 611], "fp8"),
    ("fp8_d64_g8_s32", 1, 16, 2, 64, 32, [1777], "fp8"),
    ("fp8_d128_g2_s64", 2, 4, 2, 128, 64, [2048, 97], "fp8"),
    ("f32_d64_g4_s16", 2, 8, 2, 64, 16, [515, 1024], "f32"),
    ("f32_d128_g2_s32", 1, 4, 2, 128, 32, [700], "f32"),
]


@pytest.fixture(scope="module", params=CASES, ids=[c[0] for c in CASES])
def small_case(request):
    name, B, Hq, Hkv, d, S, lens, dt = request.param
    w = wl.Workload(name, B, Hq, Hkv, d, max(lens), S, 8, dt, seed=100 + len(name), seq_lens=lens)
    inp = wl.make_inputs(w, "cuda")
    q, kv = oracle_view(inp)
    return w, inp, q[0], kv


def _random_sets(w, rng, sizes):
    """Disjoint P, M per unit with the requested sizes (clipped to the number of blocks)."""
    P, M = [], []
    for b in range(w.batch):
        prow, mrow = [], []
        nb = w.blocks_of(b)
        for h in range(w.num_kv_heads):
            n_p, n_m = sizes[(b * w.num_kv_heads + h) % len(sizes)]
            perm = rng.permutation(nb)
            n_p = min(n_p, nb)
            n_m = min(n_m, nb - n_p)
            prow.append(list(perm[:n_p]))
            mrow.append(list(perm[n_p:n_p + n_m]))
        P.append(prow)
        M.append(mrow)
    return P, M


def test_spec_then_repair_equals_union(small_case):
    w, inp, q, kv = small_case
    rng = np.random.default_rng(1)
    P, M = _random_sets(w, rng, [(5, 3), (0, 4), (7, 0), (1, 1), (11, 9)])
    dkv = device_kv(inp)
    cap = 24
    Pd, Md = sets_to_device(P, cap), sets_to_device(M, cap)
    state = bd.spec_attn(inp.q[0], dkv, w.block, Pd, w.scale)
    assert_heads(state, orc.spec_states(q, kv, w.block, P, w.scale), "spec")
    out = torch.empty_like(state.acc)
    bd.repair(inp.q[0], dkv, w.block, Md, w.scale, state, out=out)
    union = [[sorted(set(P[b][h]) | set(M[b][h])) for h in range(w.num_kv_heads)] for b in range(w.batch)]
    ref = orc.spec_states(q, kv, w.block, union, w.scale)
    assert_heads(state, ref, "repair")
    o = out.double().cpu().numpy()
    for (b, h), st in ref.items():
        assert np.max(np.abs(o[b, h] - st.out)) <= 5e-3


def test_select_spec_matches_separate_calls(small_case):
    """The fused launch computes what prr_select and prr_spec_attn compute: scores, A and M bit for bit,
    the state bit for bit (same chunking and merge order) and within tolerance of the oracle."""
    w, inp, q, kv = small_case
    rng = np.random.default_rng(5)
    P, _ = _random_sets(w, rng, [(5, 0), (0, 0), (7, 0), (1, 0), (11, 0)])
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    Pd = sets_to_device(P, 16)
    for kk in (0, 3, 8, 64):
        scores, A, M = bd.select(inp.q[0], dkv, meta, w.block, kk, P=Pd)
        state = bd.spec_attn(inp.q[0], dkv, w.block, Pd, w.scale)
        fs, fA, fM, fstate = bd.select_spec(inp.q[0], dkv, meta, w.block, kk, Pd, w.scale)
        assert torch.equal(fs, scores)
        assert fA.lists() == A.lists() and fM.lists() == M.lists()
        for name in ("acc", "l", "m"):
            assert torch.equal(getattr(fstate, name), getattr(state, name)), name
    assert_heads(fstate, orc.spec_states(q, kv, w.block, P, w.scale), "fused spec")


def test_empty_missed_set_leaves_state_bitwise(small_case):
    w, inp, q, kv = small_case
    rng = np.random.default_rng(2)
    P, _ = _random_sets(w, rng, [(6, 0)])
    dkv = device_kv(inp)
    state = bd.spec_attn(inp.q[0], dkv, w.block, sets_to_device(P, 8), w.scale)
    before = state.clone()
    empty = bd.BlockSet.empty(w.batch, w.num_kv_heads, 8)
    out = torch.full_like(state.acc, 7.0)
    bd.repair(inp.q[0], dkv, w.block, empty, w.scale, state, out=out)
    torch.cuda.synchronize()
    assert torch.equal(state.acc, before.acc) and torch.equal(state.l, before.l)
    assert torch.equal(state.m, before.m)
    assert torch.allclose(out, before.acc / before.l[..., None], rtol=1e-6, atol=0)


def test_empty_speculation_is_plain_dsa(small_case):
    w, inp, q, kv = small_case
    rng = np.random.default_rng(3)
    A, _ = _random_sets(w, rng, [(8, 0), (3, 0)])
    dkv = device_kv(inp)
    empty = bd.BlockSet.empty(w.batch, w.num_kv_heads, 8)
    state = bd.spec_attn(inp.q[0], dkv, w.block, empty, w.scale)
    torch.cuda.synchronize()
    assert torch.all(state.l == 0) and torch.all(state.m == -math.inf) and torch.all(state.acc == 0)
    bd.repair(inp.q[0], dkv, w.block, sets_to_device(A, 8), w.scale, state)
    assert_heads(state, orc.spec_states(q, kv, w.block, A, w.scale), "dsa")


def test_order_independence_and_determinism(small_case):
    w, inp, q, kv = small_case
    rng = np.random.default_rng(4)
    P, _ = _random_sets(w, rng, [(9, 0)])
    dkv = device_kv(inp)
    s1 = bd.spec_attn(inp.q[0], dkv, w.block, sets_to_device(P, 12), w.scale)
    s2 = bd.spec_attn(inp.q[0], dkv, w.block, sets_to_device(P, 12), w.scale)
    torch.cuda.synchronize()
    assert torch.equal(s1.acc, s2.acc) and torch.equal(s1.l, s2.l) and torch.equal(s1.m, s2.m)
    shuffled = [[list(rng.permutation(p)) for p in row] for row in P]
    s3 = bd.spec_attn(inp.q[0], dkv, w.block, sets_to_device(shuffled, 12), w.scale)
    ref = orc.spec_states(q, kv, w.block, P, w.scale)
    assert_heads(s3, ref, "shuffled")
    # two repairs in sequence equal one repair with the union
    P2, M2 = _random_sets(w, rng, [(3, 6)])
    half = [[m[: len(m) // 2] for m in row] for row in M2]
    rest = [[m[len(m) // 2:] for m in row] for row in M2]
    st = bd.spec_attn(inp.q[0], dkv, w.block, sets_to_device(P2, 12), w.scale)
    bd.repair(inp.q[0], dkv, w.block, sets_to_device(half, 12), w.scale, st)
    bd.repair(inp.q[0], dkv, w.block, sets_to_device(rest, 12), w.scale, st)
    union = [[sorted(set(P2[b][h]) | set(M2[b][h])) for h in range(w.num_kv_heads)] for b in range(w.batch)]
    assert_heads(st, orc.spec_states(q, kv, w.block, union, w.scale), "two repairs")


def test_meta_scores_topk(small_case):
    w, inp, q, kv = small_case
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    ometa = orc.build_meta(kv, w.block, w.num_kv_heads)
    gm = _meta_bits(meta, w)
    for kk in (0, 1, 5, 8, 64):      # 64 exceeds every case's block count: A = all blocks
        A = bd.BlockSet.empty(w.batch, w.num_kv_heads, max(1, kk))
        scores, A, _ = bd.select(inp.q[0], dkv, meta, w.block, kk, A=A)
        osc, oA, _ = orc.select(q, ometa, w.group, kk)
        gs = scores.cpu().numpy()
        got = A.lists()
        for b in range(w.batch):
            nb = w.blocks_of(b)
            for h in range(w.num_kv_heads):
                assert np.array_equal(gm[b, h, :, 0, :nb].T, ometa[b][h][0])
                assert np.array_equal(gm[b, h, :, 1, :nb].T, ometa[b][h][1])
                assert np.array_equal(gs[b, h, :nb], osc[b][h]), (b, h)
                assert got[b][h] == list(oA[b][h]), (kk, b, h)


def test_select_ties_go_to_smaller_index():
    """Identical keys in every block give equal scores everywhere: A must be the first K blocks,
    and M = A minus P in ascending order."""
    w = wl.Workload("ties", 1, 4, 1, 64, 16 * 40, 16, 7, "bf16", seed=7, shuffle_pages=False)
    inp = wl.make_inputs(w, "cuda")
    inp.k_cache[:] = inp.k_cache[0:1, :, 0:1, :].clone()
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    P = sets_to_device([[[3, 9, 0, 30]]], 8)
    scores, A, M = bd.select(inp.q[0], dkv, meta, w.block, w.topk, P=P)
    s = scores[0, 0, :40].cpu().numpy()
    assert np.all(s == s[0])
    assert A.lists()[0][0] == list(range(7))
    assert M.lists()[0][0] == [1, 2, 4, 5, 6]


# --------------------------------------------------------------------------------------------------
# Multi-step predictor trajectory (reduced 128K workload) with births
# --------------------------------------------------------------------------------------------------


def test_predictor_trajectory_bit_exact():
    w = wl.scaled(wl.C3, name="c3_small", batch=2, context=16384, steps=12, topk=16,
                  seq_lens=[16384, 12000])
    inp = wl.make_inputs(w, "cuda")
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    nmax = bd.max_blocks(dkv, w.block)
    B, H = w.batch, w.num_kv_heads
    level = torch.zeros((B, H, nmax), dtype=torch.float64, device="cuda")
    trend = torch.zeros_like(level)
    live = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    alpha, beta, gamma = w.ema
    views = {(b, h): unit_view(inp, b, h) for b in range(B) for h in range(H)}
    metas = {k: unit_meta(v[1], w.block) for k, v in views.items()}
    olevel = {k: np.zeros(0) for k in views}
    otrend = {k: np.zeros(0) for k in views}
    olive = {k: 0 for k in views}
    P = bd.BlockSet.empty(B, H, w.topk)
    oP = {k: np.zeros(0, dtype=np.int64) for k in views}
    # lengths grow by one block every 4 steps for sequence 1 (new blocks are born)
    lens = list(w.lengths)
    for t in range(w.steps):
        if t and t % 4 == 0:
            lens[1] = min(lens[1] + w.block, w.context)
            inp.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))
            bd.build_meta(dkv, w.block, meta)      # the grown sequence's blocks get metadata
            for h in range(H):
                metas[(1, h)] = unit_meta(unit_view(inp, 1, h, length=lens[1])[1], w.block)
        scores, A, M = bd.select(inp.q[t], dkv, meta, w.block, w.topk, P=P)
        Pn = bd.predict(scores, inp.seq_len, w.block, alpha, beta, gamma, w.topk, level, trend, live)
        gs, gA, gM, gP = scores.cpu().numpy(), A.lists(), M.lists(), Pn.lists()
        gl, gt = level.cpu().numpy(), trend.cpu().numpy()
        for (b, h), (qv, kvv) in views.items():
            nb = -(-lens[b] // w.block)
            mn, mx = metas[(b, h)]
            qv_t = orc.upcast(wl.to_numpy_bits(inp.q[t, b, h * w.group:(h + 1) * w.group]), w.dtype)[None]
            s = orc.quest_scores(orc.representative_query(qv_t, 0, 0, w.group), mn[:nb], mx[:nb])
            a = orc.topk_blocks(s, w.topk)
            assert np.array_equal(gs[b, h, :nb], s), (t, b, h)
            assert gA[b][h] == list(a), (t, b, h)
            assert gM[b][h] == list(orc.set_minus(a, oP[(b, h)])), (t, b, h)
            lv, tr, lvn, pn = orc.predict_step(olevel[(b, h)], otrend[(b, h)], olive[(b, h)], s, alpha, beta,
                                               gamma, w.topk)
            olevel[(b, h)], otrend[(b, h)], olive[(b, h)], oP[(b, h)] = lv, tr, lvn, pn
            assert np.array_equal(gl[b, h, :nb], lv) and np.array_equal(gt[b, h, :nb], tr), (t, b, h)
            assert gP[b][h] == list(pn), (t, b, h)
        P = Pn
    assert live.cpu().numpy().tolist() == [[-(-l // w.block)] * H for l in lens]


@pytest.mark.parametrize("nblocks,topk", [(300, 40), (900, 40), (1024, 40), (1025, 40), (2048, 40), (2049, 40),
                                         (4097, 40), (8192, 128), (4096, 600), (8192, 600), (16384, 300),
                                         (32768, 400), (32768, 512), (33000, 256)])
def test_select_spec_fused_topk_shapes(nblocks, topk):
    """The fused launch's top-K runs in the last scoring workgroup: over all scores with 1, 2 or 4 keys
    per thread (units of up to 1024 blocks), and beyond that in two stages (local top-min(K, 512)
    candidates of every scoring workgroup, then the top-K of the candidates, up to 16 per thread; K = 600
    caps the local candidates at 512; 1025 blocks leave one block in the last part).  With more than 4096
    candidate slots (8192 blocks at K = 600, 16384 at K = 300) a third stage follows: groups of parts (up
    to 2048 candidate slots) keep their top-K, and the unit's last group ranks the groups' candidates,
    inside the launch (its scoring workgroups are resident); rows of 32768 blocks and more score in
    1024-block parts, and at 32768 blocks with K = 512, groups of up to 4096 slots keep the last ranking
    within 4096 slots; 33000 blocks (above one ranking's P bitmap) leave 232 blocks in the last part.
    Every shape against the separate calls (bit for bit) and the oracle's scores and sets."""
    lens = [nblocks * 16, nblocks * 16 - 37]
    w = wl.Workload(f"fused_{nblocks}", 2, 8, 2, 64, max(lens), 16, topk, "bf16", seed=900 + nblocks,
                    seq_lens=lens)
    inp = wl.make_inputs(w, "cuda")
    q, kv = oracle_view(inp)
    q = q[0]
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    rng = np.random.default_rng(nblocks)
    P, _ = _random_sets(w, rng, [(30, 0), (0, 0), (40, 0), (7, 0)])
    Pd = sets_to_device(P, 48)
    assert w.topk <= 600
    scores, A, M = bd.select(inp.q[0], dkv, meta, w.block, w.topk, P=Pd)
    state = bd.spec_attn(inp.q[0], dkv, w.block, Pd, w.scale)
    fs, fA, fM, fstate = bd.select_spec(inp.q[0], dkv, meta, w.block, w.topk, Pd, w.scale)
    # a second call on the same workspace: the arrival counters were left at zero
    ws = bd.select_spec_workspace_for(dkv, w.num_q_heads, w.block, w.topk, Pd.cap)
    for _ in range(2):
        fs2, fA2, fM2, fstate2 = bd.select_spec(inp.q[0], dkv, meta, w.block, w.topk, Pd, w.scale, ws=ws)
        assert fA2.lists() == A.lists() and fM2.lists() == M.lists()
    assert torch.equal(fs, scores) and torch.equal(fs2, scores)
    assert fA.lists() == A.lists() and fM.lists() == M.lists()
    for name in ("acc", "l", "m"):
        assert torch.equal(getattr(fstate, name), getattr(state, name)), name
    ometa = orc.build_meta(kv, w.block, w.num_kv_heads)
    osc, oA, _ = orc.select(q, ometa, w.group, w.topk)
    gs = fs.cpu().numpy()
    got_a, got_m = fA.lists(), fM.lists()
    for b in range(w.batch):
        nb = w.blocks_of(b)
        for h in range(w.num_kv_heads):
            assert np.array_equal(gs[b, h, :nb], osc[b][h]), (b, h)
            assert got_a[b][h] == list(oA[b][h]), (b, h)
            assert got_m[b][h] == list(orc.set_minus(oA[b][h], P[b][h])), (b, h)
    assert_heads(fstate, orc.spec_states(q, kv, w.block, P, w.scale), "fused spec")


def test_select_spec_with_more_scoring_workgroups_than_cus():
    """Many units (64 sequences x 8 kv heads, one scoring workgroup each): the scoring workgroups alone
    outnumber the CUs, so the fused launch spreads the speculative pass over the remaining slots with
    longer chunks than prr_spec_attn uses.  Scores, A and M stay bit for bit; the state matches the
    separate call within the parity tolerance and the oracle on sampled units."""
    lens = wl.ragged_lengths(wl.Workload("many_units", 64, 32, 8, 128, 2048, 16, 8, "bf16", seed=41), 900, 2048)
    w = wl.Workload("many_units", 64, 32, 8, 128, max(lens), 16, 16, "bf16", seed=41, seq_lens=lens)
    inp = wl.make_inputs(w, "cuda")
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    rng = np.random.default_rng(7)
    P, _ = _random_sets(w, rng, [(40, 0), (0, 0), (90, 0), (3, 0), (128, 0)])
    Pd = sets_to_device(P, 128)
    scores, A, M = bd.select(inp.q[0], dkv, meta, w.block, w.topk, P=Pd)
    state = bd.spec_attn(inp.q[0], dkv, w.block, Pd, w.scale)
    fs, fA, fM, fstate = bd.select_spec(inp.q[0], dkv, meta, w.block, w.topk, Pd, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(fs, scores)
    assert fA.lists() == A.lists() and fM.lists() == M.lists()
    a1, a2 = state.acc.double(), fstate.acc.double()
    l1, l2 = state.l.double(), fstate.l.double()
    m1, m2 = state.m.double(), fstate.m.double()
    assert torch.equal(l1 == 0, l2 == 0)
    live = l1 > 0
    assert torch.all((l1[live] - l2[live]).abs() <= 1e-4 * l1[live])
    assert torch.all((m1[live] - m2[live]).abs() <= 1e-4 * torch.clamp(m1[live].abs(), min=1.0))
    o1 = a1[live] / l1[live][:, None]
    o2 = a2[live] / l2[live][:, None]
    assert float((o1 - o2).abs().max()) <= 5e-3
    for b, h in ((0, 0), (17, 2), (63, 7)):
        q, kv = unit_view(inp, b, h)
        for g in range(w.group):
            ref = orc.head_state(q, kv, 0, g, w.group, sorted(P[b][h]), w.block, w.scale)
            hq = h * w.group + g
            assert_state(fstate.acc[b, hq].double().cpu().numpy(), float(fstate.l[b, hq]), float(fstate.m[b, hq]),
                         ref, f"fused b={b} kvh={h} g={g}")
