"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Each case runs the library on the whole workload and checks a sample of (sequence, kv head) units
against the oracle, one unit at a time: block metadata rows, Quest scores, the sets A, M and P (bit
for bit), the EMA state (bit for bit), and the attention state (O within 5e-3, l and m within 1e-4
relative).  Sizes:
  * Llama-3-8B-shaped layer: 32K context, batch 1, 32q/8kv, block 16, K = 128, 32 planted blocks;
  * 128K context, batch 8, block 64, K = 64: all 64 layer steps of the EMA-driven trajectory (the steps
    bench.py times);
  * 512K context, 16-token pages in random physical order, block 16 (32768 blocks), K = 256;
  * 70B-shaped share: 256K context, batch 4, 64q/8kv (G = 8), block 32, K = 128: all 16 layer steps with
    the EMA parameters theta* that calibration of its 8192 x 512 prefill matrix selects (the oracle's
    stored result, which the calibration tests hold the GPU to).
"""
import json
import os

import numpy as np
import pytest
import torch

from _gpu import assert_state, device_kv, require_gpu, sets_to_device, unit_meta, unit_view
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl
from block_sparse_attention_quest_amd.layer_step import PRRLayer
from oracle import prr_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


def _unit_q(inp, b, h, step):
    w = inp.w
    return orc.upcast(wl.to_numpy_bits(inp.q[step, b, h * w.group:(h + 1) * w.group]), w.dtype)[None]


_VIEWS = {"inp": None, "views": {}}


def _kv_view(inp, b, h):
    """Oracle view of unit (b, h)'s cache, cached for the current input set only (the cache holds the
    input object itself, so a new input set never sees another one's views)."""
    if _VIEWS["inp"] is not inp:
        _VIEWS["inp"], _VIEWS["views"] = inp, {}
    views = _VIEWS["views"]
    if (b, h) not in views:
        views[(b, h)] = unit_view(inp, b, h)[1]
    return views[(b, h)]


def _check_unit_attention(state: bd.AttnState, out, inp, b, h, step, blocks, what):
    """state/out heads of unit (b, h) against oracle attention over `blocks`."""
    w = inp.w
    q, kv = _unit_q(inp, b, h, step), _kv_view(inp, b, h)
    acc = state.acc.double().cpu().numpy()
    l = state.l.double().cpu().numpy()
    m = state.m.double().cpu().numpy()
    o = out.double().cpu().numpy() if out is not None else None
    for g in range(w.group):
        ref = orc.head_state(q, kv, 0, g, w.group, sorted(blocks), w.block, w.scale)
        hq = h * w.group + g
        assert_state(acc[b, hq], l[b, hq], m[b, hq], ref, f"{what} b={b} kvh={h} g={g}")
        if o is not None:
            assert np.max(np.abs(o[b, hq] - ref.out)) <= 5e-3, f"{what} out b={b} kvh={h} g={g}"


def _check_unit_selection(inp, b, h, step, meta_dev, scores_dev, A: bd.BlockSet, P_lists=None, M=None,
                          ometa=None):
    """Metadata rows, scores, A (and M) of unit (b, h) against the oracle; returns (scores, A, meta)."""
    w = inp.w
    nb = w.blocks_of(b)
    if ometa is None:
        ometa = unit_meta(_kv_view(inp, b, h), w.block)
    mn, mx = ometa
    gm = orc.upcast(wl.to_numpy_bits(meta_dev[b, h]), w.dtype) if meta_dev is not None else None
    if gm is not None:
        assert np.array_equal(gm[:, 0, :nb].T, mn) and np.array_equal(gm[:, 1, :nb].T, mx), (b, h)
    q = _unit_q(inp, b, h, step)
    s = orc.quest_scores(orc.representative_query(q, 0, 0, w.group), mn, mx)
    a = orc.topk_blocks(s, w.topk)
    assert np.array_equal(scores_dev[b, h, :nb].cpu().numpy(), s), (step, b, h)
    assert A.lists()[b][h] == list(a), (step, b, h)
    if M is not None:
        assert M.lists()[b][h] == list(orc.set_minus(a, P_lists[b][h])), (step, b, h)
    return s, a, ometa


def test_llama3_8b_layer_32k():
    w = wl.C2
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    meta = bd.build_meta(kv, w.block)
    scores, A, _ = bd.select(inp.q[0], kv, meta, w.block, w.topk)
    nb = w.blocks_of(0)
    P = [[None] * w.num_kv_heads]
    for h in range(w.num_kv_heads):
        _, a, _ = _check_unit_selection(inp, 0, h, 0, meta, scores, A)
        assert set(inp.planted[0, h].tolist()) <= set(a.tolist()), h   # planted blocks are selected
        P[0][h] = list(wl.make_spec_set(w, a, nb, w.spec_hit, w.spec_miss, salt=h))
    Pd = sets_to_device(P, w.topk)
    scores2, A2, M, state = bd.select_spec(inp.q[0], kv, meta, w.block, w.topk, Pd, w.scale)
    spec_copy = state.clone()
    out = torch.empty_like(state.acc)
    bd.repair(inp.q[0], kv, w.block, M, w.scale, state, out=out)
    torch.cuda.synchronize()
    for h in range(w.num_kv_heads):
        _, a, _ = _check_unit_selection(inp, 0, h, 0, None, scores2, A2, P, M)
        m_h = orc.set_minus(a, P[0][h])
        assert len(m_h) == w.spec_miss, h
        _check_unit_attention(spec_copy, None, inp, 0, h, 0, P[0][h], "spec")
        _check_unit_attention(state, out, inp, 0, h, 0, set(P[0][h]) | set(m_h.tolist()), "repair")


def _trajectory(w, steps, units, ema, budget=None):
    """Run `steps` layer steps through PRRLayer (the single-stream step bench.py times) and check sampled
    units against the oracle's select / spec / repair / predict, step by step.  budget: |P| in blocks
    (default K), or a list: the budget of the prediction made at each step (PRRLayer.set_budget)."""
    budget = w.topk if budget is None else budget
    budgets = list(budget) if isinstance(budget, (list, tuple)) else [budget] * steps
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    layer = PRRLayer(kv, w.num_q_heads, w.block, w.topk, budgets[0], ema=ema, scale=w.scale,
                     max_budget=max(budgets))
    alpha, beta, gamma = ema
    metas = {u: unit_meta(_kv_view(inp, *u), w.block) for u in units}
    ost = {u: (np.zeros(0), np.zeros(0), 0, np.zeros(0, dtype=np.int64)) for u in units}
    for t in range(steps):
        layer.set_budget(budgets[t])
        P_before = layer.P_cur.lists()
        out = layer.step(inp.q[t])
        torch.cuda.synchronize()
        P_after = layer.P_cur.lists()
        lv_dev, tr_dev = layer.level.cpu().numpy(), layer.trend.cpu().numpy()
        for (b, h) in units:
            lv, tr, live, P = ost[(b, h)]
            assert sorted(P_before[b][h]) == list(P), (t, b, h)
            s, a, _ = _check_unit_selection(inp, b, h, t, layer.meta if t == 0 else None, layer.scores, layer.A,
                                            P_before, layer.M, metas[(b, h)])
            m_h = orc.set_minus(a, P)
            _check_unit_attention(layer.state, out, inp, b, h, t, set(P.tolist()) | set(m_h.tolist()), f"step {t}")
            lv, tr, live, P = orc.predict_step(lv, tr, live, s, alpha, beta, gamma, budgets[t])
            nb = w.blocks_of(b)
            assert np.array_equal(lv_dev[b, h, :nb], lv) and np.array_equal(tr_dev[b, h, :nb], tr), (t, b, h)
            assert P_after[b][h] == list(P), (t, b, h)
            ost[(b, h)] = (lv, tr, live, P)
    return layer


def test_ctx128k_batch8_trajectory():
    """Every one of the 64 decode steps, on four sampled units."""
    _trajectory(wl.C3, wl.C3.steps, [(0, 0), (3, 5), (5, 2), (7, 7)], wl.C3.ema)


@pytest.mark.parametrize("select_us,want_delta", [(15.0, 0.5), (30.0, 2.0)])
def test_ctx128k_batch8_trajectory_with_planned_budget(select_us, want_delta):
    """|P| sized by the speculation-budget planner: a latency table (speculation 10 us + 9 us per unit of
    delta, selection flat at `select_us`) picks delta at 128K, and the layer runs with |P| = delta K."""
    from block_sparse_attention_quest_amd.layer_step import speculation_budget

    deltas = [0.25, 0.5, 1.0, 2.0, 3.0]
    ctx = [16384.0, 65536.0, 131072.0]
    tab = bd.BudgetTable(ctx, [select_us] * 3, deltas, [[10.0 + 9.0 * d] * 3 for d in deltas], 1)
    budget = speculation_budget(tab, wl.C3.context, wl.C3.topk)
    assert budget == int(round(want_delta * wl.C3.topk))
    _trajectory(wl.C3, 3, [(2, 3), (6, 0)], wl.C3.ema, budget)


def test_ctx128k_batch8_trajectory_with_budget_changes():
    """|P| changed between steps (as a planner would when the context grows): 64, then 128, then 32
    blocks, with sets and workspaces sized once for the largest."""
    _trajectory(wl.C3, 4, [(1, 6), (4, 2)], wl.C3.ema, [64, 128, 32, 64])


def test_ctx512k_trajectory_with_budgets_above_341():
    """32768 blocks per row (512K at 16-token blocks) with |P| above 341, where the predictor's ranking
    takes groups of 4096 candidate slots, and its workspace is sized over every budget the layer may use:
    |P| = 400, 342, then 256, against the oracle step by step."""
    w = wl.scaled(wl.C4, name="ctx512k_traj", steps=3, drift_rho=0.9, query_mean_gain=0.64)
    _trajectory(w, 3, [(0, 1), (0, 6)], wl.C3.ema, [400, 342, 256])


def test_ctx128k_batch8_fp8_trajectory():
    """The same workload with an fp8 (E4M3) cache, as `bench.py --kv-dtype fp8` runs it."""
    _trajectory(wl.scaled(wl.C3, dtype="fp8"), 3, [(1, 1), (6, 4)], wl.C3.ema)


def test_ctx512k_paged_selection_and_repair():
    w = wl.C4
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    meta = bd.build_meta(kv, w.block)
    scores, A, _ = bd.select(inp.q[0], kv, meta, w.block, w.topk)
    nb = w.blocks_of(0)
    units = [0, 5]
    P = [[list(range(w.spec_hit + w.spec_miss)) for _ in range(w.num_kv_heads)]]   # placeholders
    ometas = {}
    for h in units:
        _, a, ometas[h] = _check_unit_selection(inp, 0, h, 0, meta, scores, A)
        P[0][h] = list(wl.make_spec_set(w, a, nb, w.spec_hit, w.spec_miss, salt=h))
    Pd = sets_to_device(P, w.topk)
    scores2, A2, M, state = bd.select_spec(inp.q[0], kv, meta, w.block, w.topk, Pd, w.scale)
    spec_copy = state.clone()
    out = torch.empty_like(state.acc)
    bd.repair(inp.q[0], kv, w.block, M, w.scale, state, out=out)
    torch.cuda.synchronize()
    for h in units:
        _, a, _ = _check_unit_selection(inp, 0, h, 0, None, scores2, A2, P, M, ometas[h])
        m_h = orc.set_minus(a, P[0][h])
        assert len(m_h) == w.spec_miss
        _check_unit_attention(spec_copy, None, inp, 0, h, 0, P[0][h], "spec")
        _check_unit_attention(state, out, inp, 0, h, 0, set(P[0][h]) | set(m_h.tolist()), "repair")


def test_llama70b_share_calibrated_trajectory():
    """All 16 steps with theta* of the calibration (the GPU's choice, which must be the oracle's stored
    one), on three sampled units."""
    w = wl.C5
    gold = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                       "calibration_c5_8192x512.json")))
    IS = wl.make_calibration_scores(w)
    H, best = bd.calibrate(torch.from_numpy(IS).cuda(), w.topk)
    j = int(best.cpu().numpy()[0])
    assert j == gold["best"], (j, gold["best"])
    ema = tuple(float(x) for x in bd.calibration_grid("cpu").numpy()[j])
    print(f"[c5] theta* = {ema}", flush=True)
    _trajectory(w, w.steps, [(0, 0), (2, 6), (3, 3)], ema)


def test_two_stream_schedule_matches_one_stream():
    """The pages' three-stream schedule and the single-stream step of the same calls (select_spec, repair,
    predict) give the same sets, predictor state and output, bit for bit, over a few steps of the 128K
    batch-8 trajectory (reduced to 32K); the layer step as one launch gives the same sets and predictor
    state bit for bit and the output within the tolerance (its partial states merge in another grouping)."""
    w = wl.scaled(wl.C3, name="c3_32k", context=32768, steps=5)
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    a = PRRLayer(kv, w.num_q_heads, w.block, w.topk, w.topk, ema=w.ema, scale=w.scale, fused=False)
    b = PRRLayer(kv, w.num_q_heads, w.block, w.topk, w.topk, ema=w.ema, scale=w.scale, fused=False)
    c = PRRLayer(kv, w.num_q_heads, w.block, w.topk, w.topk, ema=w.ema, scale=w.scale)
    for t in range(w.steps):
        oa = a.step(inp.q[t]).clone()
        ob = b.step_two_streams(inp.q[t]).clone()
        oc = c.step(inp.q[t])
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), t
        assert a.A.lists() == b.A.lists() == c.A.lists() and a.M.lists() == b.M.lists() == c.M.lists(), t
        assert a.P_cur.lists() == b.P_cur.lists() == c.P_cur.lists(), t
        assert torch.equal(a.level, b.level) and torch.equal(a.trend, b.trend), t
        assert torch.equal(a.level, c.level) and torch.equal(a.trend, c.trend), t
        for name in ("acc", "l", "m"):
            assert torch.equal(getattr(a.state, name), getattr(b.state, name)), (t, name)
        assert float((oa - oc).abs().max()) <= 5e-3, t


@pytest.mark.parametrize("dtype,hq,d", [("bf16", 8, 64), ("fp8", 16, 128), ("bf16", 64, 128)],
                         ids=["bf16_g2_d64", "fp8_g4_d128", "bf16_g16_d128"])
def test_largest_chunks_and_several_chunks_per_workgroup(dtype, hq, d):
    """Sets of thousands of blocks: chunks reach their 256-page maximum (64 pages per wave, the longest
    tile walk), and a unit has more chunks than the launch has workgroups, so workgroups walk several
    chunks in turn - the speculative pass for units with a large P, repair for units with a large M.
    Sampled units of both kinds against the oracle."""
    w = wl.Workload("big_sets", 4, hq, 4, d, 81920, 16, 8, dtype, seed=321)
    inp = wl.make_inputs(w, "cuda")
    dkv = device_kv(inp)
    nb = w.blocks_of(0)
    cap = 4800
    rng = np.random.default_rng(9)
    P, M = [], []
    for b in range(w.batch):
        prow, mrow = [], []
        for h in range(w.num_kv_heads):
            u = b * w.num_kv_heads + h
            n_p, n_m = (cap - 13 * u, 300) if u % 2 == 0 else (200, cap - 13 * u)
            perm = rng.permutation(nb)
            prow.append(sorted(perm[:n_p].tolist()))
            mrow.append(sorted(perm[n_p:n_p + n_m].tolist()))
        P.append(prow)
        M.append(mrow)
    print(f"[big sets] {dtype} G={w.group} d={d} B={w.batch} kv heads={w.num_kv_heads} blocks={nb} cap={cap}",
          flush=True)
    state = bd.spec_attn(inp.q[0], dkv, w.block, sets_to_device(P, cap), w.scale)
    spec = state.clone()
    out = torch.empty_like(state.acc)
    bd.repair(inp.q[0], dkv, w.block, sets_to_device(M, cap), w.scale, state, out=out)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (0, 1), (3, 3), (2, 2)):
        _check_unit_attention(spec, None, inp, b, h, 0, P[b][h], "spec")
        _check_unit_attention(state, out, inp, b, h, 0, set(P[b][h]) | set(M[b][h]), "repair")
