"""GPU parity for rows longer than one top-K workgroup holds (more than 32768 blocks per sequence and kv
head): the 1M- and 2M-token contexts of the long-context models the pages evaluate, at 16-token blocks.

Selection ranks such rows in three part-parallel stages (each scoring workgroup keeps its part's local
top-K, groups of parts keep theirs, then one ranking per unit), and the predictor updates them in 512-block
parts.  The results must still be the exact top-K: scores, A, M and P bit for bit against the oracle's
brute-force ranking, the EMA state bit for bit, and the attention state within the bf16 tolerance, on
sampled units.
"""
import numpy as np
import pytest
import torch

from _gpu import assert_state, device_kv, require_gpu, sets_to_device, unit_meta, unit_view
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

pytestmark = pytest.mark.gpu

# 1M tokens, 8 kv heads (Llama-3-8B-shaped), 65536 blocks of 16 tokens, K = 256 blocks (4096 tokens)
W1M = wl.scaled(wl.C4, name="ctx1m_paged", context=1 << 20, seed=41)
# 2M tokens, 2 kv heads (a share of the heads), 131072 blocks of 16 tokens: the longest rows supported
W2M = wl.scaled(wl.C4, name="ctx2m_paged", context=1 << 21, num_q_heads=8, num_kv_heads=2, seed=42)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


def _say(msg):
    print(f"[long rows] {msg}", flush=True)


class _Unit:
    """Oracle view of one (sequence, kv head) unit: its cache, metadata, and query."""

    def __init__(self, inp, b, h, mean=False):
        self.b, self.h = b, h
        w = inp.w
        self.q, self.kv = unit_view(inp, b, h)
        if mean:
            self.meta = orc.build_mean_meta(self.kv, w.block, 1)[0][0]
        else:
            self.meta = unit_meta(self.kv, w.block)
        qbar = orc.representative_query(self.q, 0, 0, w.group)
        if mean:
            self.scores = orc.mean_scores(qbar, self.meta)
        else:
            self.scores = orc.quest_scores(qbar, *self.meta)
        self.A = orc.topk_blocks(self.scores, w.topk)


def _check_selection(w, u: _Unit, scores_dev, A: bd.BlockSet, M=None, P=None):
    nb = w.blocks_of(u.b)
    assert np.array_equal(scores_dev[u.b, u.h, :nb].cpu().numpy(), u.scores), (u.b, u.h)
    assert A.lists()[u.b][u.h] == list(u.A), (u.b, u.h)
    if M is not None:
        assert M.lists()[u.b][u.h] == list(orc.set_minus(u.A, P)), (u.b, u.h)


def _check_attention(w, u: _Unit, state: bd.AttnState, out, blocks, what):
    acc = state.acc.double().cpu().numpy()
    l = state.l.double().cpu().numpy()
    m = state.m.double().cpu().numpy()
    o = out.double().cpu().numpy() if out is not None else None
    for g in range(w.group):
        ref = orc.head_state(u.q, u.kv, 0, g, w.group, sorted(blocks), w.block, w.scale)
        hq = u.h * w.group + g
        assert_state(acc[u.b, hq], l[u.b, hq], m[u.b, hq], ref, f"{what} b={u.b} kvh={u.h} g={g}")
        if o is not None:
            assert np.max(np.abs(o[u.b, hq] - ref.out)) <= 5e-3, f"{what} out b={u.b} kvh={u.h} g={g}"


@pytest.mark.parametrize("w,heads", [(W1M, [0, 5]), (W2M, [1])], ids=["1m_65536_blocks", "2m_131072_blocks"])
def test_long_row_select_spec_repair_layer_step(w, heads):
    """prr_select, prr_select_spec (+ prr_repair) and prr_layer_step on rows of 65536 and 131072 blocks."""
    nb = w.blocks_of(0)
    assert w.max_blocks == nb and nb > 32768
    _say(f"{w.name}: inputs ({nb} blocks per row, K = {w.topk})")
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    meta = bd.build_meta(kv, w.block)
    _say(f"{w.name}: prr_select")
    scores, A, _ = bd.select(inp.q[0], kv, meta, w.block, w.topk)
    torch.cuda.synchronize()
    units = {h: _Unit(inp, 0, h) for h in heads}
    P = [[list(range(w.spec_hit + w.spec_miss)) for _ in range(w.num_kv_heads)]]   # placeholders elsewhere
    for h, u in units.items():
        gm = orc.upcast(wl.to_numpy_bits(meta[0, h]), w.dtype)
        assert np.array_equal(gm[:, 0, :nb].T, u.meta[0]) and np.array_equal(gm[:, 1, :nb].T, u.meta[1]), h
        _check_selection(w, u, scores, A)
        P[0][h] = list(wl.make_spec_set(w, u.A, nb, w.spec_hit, w.spec_miss, salt=h))
    Pd = sets_to_device(P, w.topk)
    _say(f"{w.name}: prr_select_spec + prr_repair")
    scores2, A2, M, state = bd.select_spec(inp.q[0], kv, meta, w.block, w.topk, Pd, w.scale)
    spec_copy = state.clone()
    out = torch.empty_like(state.acc)
    bd.repair(inp.q[0], kv, w.block, M, w.scale, state, out=out)
    torch.cuda.synchronize()
    for h, u in units.items():
        _check_selection(w, u, scores2, A2, M, P[0][h])
        m_h = orc.set_minus(u.A, P[0][h])
        assert len(m_h) == w.spec_miss, h
        _check_attention(w, u, spec_copy, None, P[0][h], "spec")
        _check_attention(w, u, state, out, set(P[0][h]) | set(m_h.tolist()), "repair")
    _say(f"{w.name}: prr_layer_step")
    B, H = w.batch, w.num_kv_heads
    scores3 = torch.zeros_like(scores)
    A3, M3 = bd.BlockSet.empty(B, H, w.topk), bd.BlockSet.empty(B, H, w.topk)
    st3 = bd.AttnState.empty(B, w.num_q_heads, w.head_dim)
    out3 = torch.empty_like(st3.acc)
    bd.layer_step(inp.q[0], kv, meta, w.block, w.topk, Pd, w.scale, scores3, A3, M3, st3, out=out3)
    torch.cuda.synchronize()
    assert torch.equal(scores3, scores2) and A3.lists() == A2.lists() and M3.lists() == M.lists()
    for h, u in units.items():
        m_h = orc.set_minus(u.A, P[0][h])
        _check_attention(w, u, st3, out3, set(P[0][h]) | set(m_h.tolist()), "layer step")


# Ragged rows of 40001 and 33001 blocks at K = 512 (2 sequences, 2 kv heads): neither row is a whole
# number of scoring parts, and K = 512 takes groups of 8 parts (K = 512 at these lengths has a plan only
# with 1024-block parts)
WRAG = wl.scaled(wl.C4, name="ragged_long_k512", batch=2, num_q_heads=8, num_kv_heads=2,
                 seq_lens=[40001 * 16 - 7, 33001 * 16 - 2], topk=512, spec_hit=348, spec_miss=164, seed=44)


def test_ragged_long_rows_k512():
    """prr_select (staged), prr_select_spec + prr_repair and prr_layer_step on ragged rows of more than
    32768 blocks at K = 512: scores, A and M bit for bit and the states within tolerance on a unit of each
    sequence; the three calls agree with each other bit for bit on every unit."""
    w = WRAG
    assert [w.blocks_of(b) for b in range(w.batch)] == [40001, 33001]
    _say(f"{w.name}: inputs ({w.max_blocks} blocks max, K = {w.topk})")
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    meta = bd.build_meta(kv, w.block)
    ws = bd.select_workspace_for(kv, w.block, w.topk)
    assert ws is not None
    _say(f"{w.name}: prr_select")
    scores, A, _ = bd.select(inp.q[0], kv, meta, w.block, w.topk, ws=ws)
    torch.cuda.synchronize()
    units = [_Unit(inp, 0, 1), _Unit(inp, 1, 0)]
    P = [[None] * w.num_kv_heads for _ in range(w.batch)]
    al = A.lists()
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            P[b][h] = list(wl.make_spec_set(w, np.array(al[b][h]), w.blocks_of(b), w.spec_hit, w.spec_miss,
                                            salt=10 * b + h))
    for u in units:
        _check_selection(w, u, scores, A)
    Pd = sets_to_device(P, w.topk)
    _say(f"{w.name}: prr_select_spec + prr_repair")
    scores2, A2, M, state = bd.select_spec(inp.q[0], kv, meta, w.block, w.topk, Pd, w.scale)
    spec_copy = state.clone()
    out = torch.empty_like(state.acc)
    bd.repair(inp.q[0], kv, w.block, M, w.scale, state, out=out)
    torch.cuda.synchronize()
    assert torch.equal(scores2, scores) and A2.lists() == A.lists()
    for u in units:
        p_u = P[u.b][u.h]
        _check_selection(w, u, scores2, A2, M, p_u)
        m_u = orc.set_minus(u.A, p_u)
        assert len(m_u) == w.spec_miss, (u.b, u.h)
        _check_attention(w, u, spec_copy, None, p_u, "spec")
        _check_attention(w, u, state, out, set(p_u) | set(m_u.tolist()), "repair")
    _say(f"{w.name}: prr_layer_step")
    B, H = w.batch, w.num_kv_heads
    scores3 = torch.zeros_like(scores)
    A3, M3 = bd.BlockSet.empty(B, H, w.topk), bd.BlockSet.empty(B, H, w.topk)
    st3 = bd.AttnState.empty(B, w.num_q_heads, w.head_dim)
    out3 = torch.empty_like(st3.acc)
    bd.layer_step(inp.q[0], kv, meta, w.block, w.topk, Pd, w.scale, scores3, A3, M3, st3, out=out3)
    torch.cuda.synchronize()
    assert torch.equal(scores3, scores2) and A3.lists() == A2.lists() and M3.lists() == M.lists()
    for u in units:
        p_u = P[u.b][u.h]
        m_u = orc.set_minus(u.A, p_u)
        _check_attention(w, u, st3, out3, set(p_u) | set(m_u.tolist()), "layer step")


def test_long_row_mean_scoring_1m():
    """Mean-pooled scoring (block means) over 65536-block rows: means, scores and A bit for bit."""
    w = wl.scaled(W1M, num_q_heads=8, num_kv_heads=2)
    nb = w.blocks_of(0)
    _say(f"mean scoring: inputs ({nb} blocks)")
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    means = bd.build_mean_meta(kv, w.block)
    scores, A, _ = bd.select(inp.q[0], kv, means, w.block, w.topk, mode="mean")
    torch.cuda.synchronize()
    u = _Unit(inp, 0, 1, mean=True)
    assert np.array_equal(means[0, 1, :, :nb].cpu().numpy().astype(np.float64).T, u.meta)
    _check_selection(w, u, scores, A)


def test_long_row_fp32_cache_select_1m():
    """An fp32 cache scores 256 blocks per workgroup, so a 65536-block row has 256 parts."""
    w = wl.scaled(W1M, dtype="f32", num_q_heads=4, num_kv_heads=1, head_dim=64, topk=64)
    nb = w.blocks_of(0)
    _say(f"fp32 cache: inputs ({nb} blocks)")
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    meta = bd.build_meta(kv, w.block)
    u = _Unit(inp, 0, 0)
    P = [[list(wl.make_spec_set(w, u.A, nb, 40, 24, salt=3))]]
    Pd = sets_to_device(P, w.topk)
    scores, A, M = bd.select(inp.q[0], kv, meta, w.block, w.topk, P=Pd)
    torch.cuda.synchronize()
    _check_selection(w, u, scores, A, M, P[0][0])
    # the fp32 layer step runs selection and the passes in turn, with selection's stages in its workspace
    st = bd.AttnState.empty(1, w.num_q_heads, w.head_dim)
    scores2 = torch.zeros_like(scores)
    A2, M2 = bd.BlockSet.empty(1, 1, w.topk), bd.BlockSet.empty(1, 1, w.topk)
    out = torch.empty_like(st.acc)
    bd.layer_step(inp.q[0], kv, meta, w.block, w.topk, Pd, w.scale, scores2, A2, M2, st, out=out)
    torch.cuda.synchronize()
    assert torch.equal(scores2, scores) and A2.lists() == A.lists() and M2.lists() == M.lists()
    m_h = orc.set_minus(u.A, P[0][0])
    _check_attention(w, u, st, out, set(P[0][0]) | set(m_h.tolist()), "fp32 layer step")


@pytest.mark.parametrize("budget", [256, 64, 8])
def test_long_row_predictor_1m(budget):
    """Three EMA steps over 65536-block rows (new blocks appear between steps: a row that grows), with the
    predictor's part-parallel plan; level, trend and P bit for bit on sampled units."""
    w = W1M
    B, H, nmax = w.batch, w.num_kv_heads, w.max_blocks
    rng = np.random.default_rng(np.random.SeedSequence([w.seed, 77, budget]))
    lengths = [nmax - 300, nmax - 17, nmax]   # blocks per step
    seq = torch.zeros(B, dtype=torch.int32, device="cuda")
    level = torch.zeros((B, H, nmax), dtype=torch.float64, device="cuda")
    trend = torch.zeros_like(level)
    live = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    ws = bd.predict_workspace_for(B, H, nmax, budget)
    assert ws is not None
    alpha, beta, gamma = w.ema
    units = [(0, 0), (0, 6)]
    ost = {u: (np.zeros(0), np.zeros(0), 0, np.zeros(0, dtype=np.int64)) for u in units}
    for t, n in enumerate(lengths):
        _say(f"predictor budget {budget}: step {t} ({n} blocks)")
        s = np.zeros((B, H, nmax))
        s[:, :, :n] = rng.lognormal(0.0, 1.0, size=(B, H, n))
        seq.fill_(n * w.block)
        P = bd.predict(torch.from_numpy(s).cuda(), seq, w.block, alpha, beta, gamma, budget, level, trend,
                       live, ws=ws)
        torch.cuda.synchronize()
        lv_dev, tr_dev, lists = level.cpu().numpy(), trend.cpu().numpy(), P.lists()
        for (b, h) in units:
            lv, tr, lvn, Pu = ost[(b, h)]
            lv, tr, lvn, Pu = orc.predict_step(lv, tr, lvn, s[b, h, :n], alpha, beta, gamma, budget)
            assert np.array_equal(lv_dev[b, h, :n], lv) and np.array_equal(tr_dev[b, h, :n], tr), (t, b, h)
            assert lists[b][h] == list(Pu), (t, b, h)
            ost[(b, h)] = (lv, tr, lvn, Pu)
        assert live.cpu().numpy().tolist() == [[n] * H]


@pytest.mark.parametrize("context,topk", [(1 << 18, 64), (1 << 19, 256)], ids=["16384_blocks_k64", "32768_blocks_k256"])
def test_staged_and_single_workgroup_selection_agree(context, topk):
    """Rows of 8193 to 32768 blocks take either ranking: one top-K workgroup per row (no workspace) or the
    part-parallel stages (with one).  Scores, A and M agree bit for bit on every unit, and with the oracle
    on a sampled one."""
    w = wl.scaled(wl.C4, name="staged_vs_single", context=context, topk=topk, seed=43)
    nb = w.blocks_of(0)
    _say(f"staged vs single workgroup: inputs ({nb} blocks, K = {topk})")
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    meta = bd.build_meta(kv, w.block)
    u = _Unit(inp, 0, 3)
    hit = min(topk // 2, 3 * topk // 4)
    P = [[list(wl.make_spec_set(w, u.A, nb, hit, topk - hit, salt=h)) for h in range(w.num_kv_heads)]]
    Pd = sets_to_device(P, topk)
    ws = bd.select_workspace_for(kv, w.block, topk)
    assert ws is not None
    s1, A1, M1 = bd.select(inp.q[0], kv, meta, w.block, topk, P=Pd, staged=False)
    s2, A2, M2 = bd.select(inp.q[0], kv, meta, w.block, topk, P=Pd, ws=ws)
    s3, A3, M3 = bd.select(inp.q[0], kv, meta, w.block, topk, P=Pd, ws=ws)   # the workspace is left ready
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(s2, s3)
    assert A1.lists() == A2.lists() == A3.lists() and M1.lists() == M2.lists() == M3.lists()
    _check_selection(w, u, s2, A2, M2, P[0][3])
