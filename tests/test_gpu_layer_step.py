"""The layer step as one launch (prr_layer_step) against the calls it stands for.

prr_layer_step computes what prr_select_spec (selection and the speculative pass over P) followed by
prr_repair (the missed blocks M = A \\ P) compute ([paper] §1 and the Figure 1 flow, §3, §4.3; [blog]
Eq. (6)): scores, A and M bit for bit, and the state over P u M, whose partial states merge in another
grouping, so it is checked against the oracle's attention over P u M with the usual tolerances (O 5e-3,
l and m 1e-4 relative) and against the two calls' state with the same bars.  The cases cover the one-launch
path (bf16 and fp8 caches, one- and two-stage top-K inside the launch), the calls' path it falls back to
(fp32 caches, rows whose ranking needs a third stage), empty P and empty M, repeated calls on one
workspace, a carried predictor step and more scoring workgroups than compute units.  After every call the
workspace's status word is zero: no repair slot gave up waiting for its M.
"""
import numpy as np
import pytest
import torch

from _gpu import assert_heads, device_kv, require_gpu, sets_to_device, unit_meta, unit_view
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


def oracle_view(inp):
    """Oracle view of the whole cache (small cases): q [steps][B][Hq][d] and the paged KV."""
    w = inp.w
    q = orc.upcast(wl.to_numpy_bits(inp.q), w.dtype)
    kv = orc.make_paged_kv(wl.to_numpy_bits(inp.k_cache), wl.to_numpy_bits(inp.v_cache),
                           wl.to_numpy_bits(inp.page_table), wl.to_numpy_bits(inp.seq_len), w.dtype)
    return q, kv


def status_word(kv, hq, block, topk, p_cap, m_cap, ws):
    """The layer-step workspace's status word (after the select_spec workspace, M's attention workspace
    and the per-unit M flags, one per 256 bytes)."""
    lib = bd.load_library()
    s = kv.struct()
    import ctypes
    off = lib.prr_select_spec_workspace_bytes(ctypes.byref(s), hq, block, topk, p_cap)
    off += lib.prr_attn_workspace_bytes(kv.batch, hq, kv.num_kv_heads, kv.head_dim, block, m_cap)
    off += kv.batch * kv.num_kv_heads * 256   # one M flag per 256 bytes
    return int(ws.buf[off:off + 4].view(torch.int32).item())


def _random_p(w, rng, sizes):
    P = []
    for b in range(w.batch):
        nb = w.blocks_of(b)
        row = []
        for h in range(w.num_kv_heads):
            n = min(sizes[(b * w.num_kv_heads + h) % len(sizes)], nb)
            row.append(sorted(rng.permutation(nb)[:n].tolist()))
        P.append(row)
    return P


def _run_both(w, inp, P, topk, p_cap, pred=None):
    """Separate calls (select, spec, repair) and the layer step on the same inputs."""
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    Pd = sets_to_device(P, p_cap)
    q = inp.q[0]
    scores, A, M = bd.select(q, dkv, meta, w.block, topk, P=Pd)
    ref = bd.spec_attn(q, dkv, w.block, Pd, w.scale)
    ref_out = torch.empty_like(ref.acc)
    bd.repair(q, dkv, w.block, M, w.scale, ref, out=ref_out)
    B, H = w.batch, w.num_kv_heads
    got = bd.AttnState.empty(B, w.num_q_heads, w.head_dim)
    got_out = torch.empty_like(got.acc)
    s2 = torch.zeros_like(scores)
    A2, M2 = bd.BlockSet.empty(B, H, max(1, topk)), bd.BlockSet.empty(B, H, max(1, topk))
    ws = bd.layer_step_workspace_for(dkv, w.num_q_heads, w.block, topk, p_cap, max(1, topk))
    outs = []
    for _ in range(2):   # a second call on the same workspace: its flags and counters were left at zero
        bd.layer_step(q, dkv, meta, w.block, topk, Pd, w.scale, s2, A2, M2, got, out=got_out, ws=ws, pred=pred)
        torch.cuda.synchronize()
        outs.append((got.acc.clone(), got.l.clone(), got.m.clone(), got_out.clone()))
        assert status_word(dkv, w.num_q_heads, w.block, topk, p_cap, max(1, topk), ws) == 0
    for x, y in zip(*outs):   # deterministic: the partial states merge in slot order
        assert torch.equal(x, y)
    assert torch.equal(s2, scores)
    assert A2.lists() == A.lists() and M2.lists() == M.lists()
    return (scores, A, M, ref, ref_out), (got, got_out)


def _check_against_oracle(w, inp, P, A_lists, M_lists, got, got_out, ref):
    q, kv = oracle_view(inp)
    union = [[sorted(set(P[b][h]) | set(M_lists[b][h])) for h in range(w.num_kv_heads)] for b in range(w.batch)]
    oref = orc.spec_states(q[0], kv, w.block, union, w.scale)
    assert_heads(got, oref, "layer step")
    assert_heads(ref, oref, "separate calls")
    o = got_out.double().cpu().numpy()
    for (b, h), st in oref.items():
        assert np.max(np.abs(o[b, h] - st.out)) <= 5e-3, (b, h)
    # the two paths' states agree to the same bars
    acc, l, m = (t.double().cpu().numpy() for t in (got.acc, got.l, got.m))
    racc, rl, rm = (t.double().cpu().numpy() for t in (ref.acc, ref.l, ref.m))
    live = rl > 0
    assert np.array_equal(l > 0, live)
    assert np.all(np.abs(l - rl)[live] <= 1e-4 * rl[live])
    assert np.all(np.abs(m - rm)[live] <= 1e-4 * np.maximum(1.0, np.abs(rm[live])))
    for b, h in zip(*np.nonzero(live)):
        assert np.max(np.abs(acc[b, h] / l[b, h] - racc[b, h] / rl[b, h])) <= 5e-3


CASES = [
    # name, B, Hq, Hkv, d, block, lens, dtype, topk, P sizes
    ("bf16_d128_g4_s16_k8", 2, 8, 2, 128, 16, [1000, 611], "bf16", 8, [5, 0, 7, 11]),
    ("bf16_d128_g4_s64_k64", 2, 8, 2, 128, 64, [8192, 5000], "bf16", 64, [40, 64, 0, 63]),
    ("bf16_d64_g8_s32_k24", 1, 16, 2, 64, 32, [20000], "bf16", 24, [20, 9]),
    ("bf16_d128_g16_s32_k16", 1, 16, 1, 128, 32, [900], "bf16", 16, [16]),
    ("bf16_d128_g1_s256_k4", 2, 4, 4, 128, 256, [8192, 7000], "bf16", 4, [3, 4, 0, 1]),
    ("fp8_d128_g4_s16_k40", 2, 8, 2, 128, 16, [16000, 9000], "fp8", 40, [30, 40, 12, 0]),
    ("fp8_d64_g8_s64_k32", 1, 16, 2, 64, 64, [40000], "fp8", 32, [32, 17]),
    ("f32_d64_g4_s16_k8", 2, 8, 2, 64, 16, [515, 1024], "f32", 8, [5, 8, 0, 2]),
    ("bf16_two_stage_k128", 1, 32, 8, 128, 16, [32768], "bf16", 128, [87, 128, 100, 0]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_step_matches_separate_calls_and_oracle(case):
    name, B, Hq, Hkv, d, S, lens, dt, topk, sizes = case
    w = wl.Workload(name, B, Hq, Hkv, d, max(lens), S, topk, dt, seed=300 + len(name), seq_lens=lens)
    inp = wl.make_inputs(w, "cuda")
    rng = np.random.default_rng(len(name))
    P = _random_p(w, rng, sizes)
    p_cap = max(1, max(sizes))
    (scores, A, M, ref, ref_out), (got, got_out) = _run_both(w, inp, P, topk, p_cap)
    _check_against_oracle(w, inp, P, A.lists(), M.lists(), got, got_out, ref)


def test_layer_step_empty_m_and_k_zero():
    """P holding all of A (M empty: the state is the speculative pass alone) and K = 0 (A and M empty)."""
    w = wl.Workload("empty_m", 2, 8, 2, 128, 4096, 64, 16, "bf16", seed=77)
    inp = wl.make_inputs(w, "cuda")
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    _, A, _ = bd.select(inp.q[0], dkv, meta, w.block, w.topk)
    P = [[sorted(set(a) | {0, 1}) for a in row] for row in A.lists()]
    (_, _, M, ref, _), (got, got_out) = _run_both(w, inp, P, w.topk, 24)
    assert all(len(m) == 0 for row in M.lists() for m in row)
    _check_against_oracle(w, inp, P, A.lists(), M.lists(), got, got_out, ref)
    (_, A0, M0, ref0, _), (got0, out0) = _run_both(w, inp, P, 0, 24)
    _check_against_oracle(w, inp, P, A0.lists(), M0.lists(), got0, out0, ref0)


def test_layer_step_with_many_units():
    """64 sequences x 8 kv heads with ragged lengths: more scoring workgroups than compute units (the
    speculative pass is spread over the slots left), and 512 units' repair slots."""
    lens = wl.ragged_lengths(wl.Workload("many_ls", 64, 32, 8, 128, 2048, 16, 16, "bf16", seed=43), 900, 4096)
    w = wl.Workload("many_ls", 64, 32, 8, 128, max(lens), 16, 16, "bf16", seed=43, seq_lens=lens)
    inp = wl.make_inputs(w, "cuda")
    rng = np.random.default_rng(4)
    P = _random_p(w, rng, [16, 9, 0, 12])
    (_, A, M, ref, ref_out), (got, got_out) = _run_both(w, inp, P, w.topk, 16)
    # sampled units against the oracle (the whole cache's oracle view is large)
    for b in (0, 17, 63):
        for h in (0, 5):
            q, kv = unit_view(inp, b, h)
            blocks = sorted(set(P[b][h]) | set(M.lists()[b][h]))
            for g in range(w.group):
                st = orc.head_state(q, kv, 0, g, w.group, blocks, w.block, w.scale)
                hq = h * w.group + g
                o = got_out[b, hq].double().cpu().numpy()
                assert np.max(np.abs(o - st.out)) <= 5e-3, (b, h, g)
                assert abs(float(got.l[b, hq]) - st.l) <= 1e-4 * st.l


@pytest.mark.parametrize("blocks,topk,dt", [(32768, 256, "bf16"), (32768, 400, "fp8"), (20000, 300, "bf16")],
                         ids=["32768_k256", "32768_k400_fp8", "20000_k300"])
def test_layer_step_three_stage_rows_in_one_launch(blocks, topk, dt):
    """Rows with more candidate slots than one ranking holds (512-block parts of min(K, 512) candidates
    each, more than 4096 in all) are ranked in three stages, all inside the launch: the last part of each
    group keeps the group's top-K and the last group ranks the unit.  Scores, A and M equal the separate
    calls' bit for bit, and the state is the oracle's over P u M."""
    lens = [blocks * 16, blocks * 16 - 1000]
    w = wl.Workload("three_ls", 2, 8, 2, 64, lens[0], 16, topk, dt, seed=91 + topk, seq_lens=lens)
    inp = wl.make_inputs(w, "cuda")
    rng = np.random.default_rng(6)
    P = _random_p(w, rng, [200, topk, 0, 37])
    (_, A, M, ref, ref_out), (got, got_out) = _run_both(w, inp, P, w.topk, topk)
    _check_against_oracle(w, inp, P, A.lists(), M.lists(), got, got_out, ref)


@pytest.mark.parametrize("topk", [40, 64, 128, 300, 512], ids=lambda k: f"k{k}")
def test_wide_parts_when_parts_outnumber_cus(topk):
    """16 sequences x 2 kv heads of up to 4608 blocks: 288 scoring parts of 512 blocks, more than the GPU
    has CUs, so the fused launches score 1024 blocks per workgroup (5 parts per row) and rank them in two
    stages with 2, 4, 8 or 16 slots per thread (K = 64, 128, 300, 512); at K = 40 (1 slot per thread) they
    keep the 512-block parts.  Scores, A and M of prr_select_spec and prr_layer_step equal prr_select's bit
    for bit, A the oracle's on sampled units, and the layer step's state the separate calls' within
    tolerance."""
    lens = [4608 * 16 - 16 * 37 * k - (k % 3) for k in range(16)]
    w = wl.Workload("many_parts", 16, 8, 2, 64, lens[0], 16, topk, "bf16", seed=300 + topk, seq_lens=lens)
    inp = wl.make_inputs(w, "cuda")
    rng = np.random.default_rng(topk)
    P = _random_p(w, rng, [topk // 2, topk, 0, 17])
    (scores, A, M, ref, ref_out), (got, got_out) = _run_both(w, inp, P, topk, topk)
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    Pd = sets_to_device(P, topk)
    s3, A3, M3, _ = bd.select_spec(inp.q[0], dkv, meta, w.block, topk, Pd, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(s3, scores) and A3.lists() == A.lists() and M3.lists() == M.lists()
    for b, h in ((0, 0), (7, 1), (15, 1)):
        q, ukv = unit_view(inp, b, h)
        mn, mx = unit_meta(ukv, w.block)
        s = orc.quest_scores(orc.representative_query(q, 0, 0, w.group), mn, mx)
        assert np.array_equal(scores[b, h, :w.blocks_of(b)].cpu().numpy(), s), (b, h)
        assert A.lists()[b][h] == list(orc.topk_blocks(s, topk)), (b, h)
    acc, l, m = (t.double().cpu().numpy() for t in (got.acc, got.l, got.m))
    racc, rl, rm = (t.double().cpu().numpy() for t in (ref.acc, ref.l, ref.m))
    live = rl > 0
    assert np.array_equal(l > 0, live)
    assert np.all(np.abs(l - rl)[live] <= 1e-4 * rl[live])
    assert np.all(np.abs(m - rm)[live] <= 1e-4 * np.maximum(1.0, np.abs(rm[live])))
    for b, h in zip(*np.nonzero(live)):
        assert np.max(np.abs(acc[b, h] / l[b, h] - racc[b, h] / rl[b, h])) <= 5e-3


def test_layer_step_carrying_a_predictor_step():
    """A predictor step of another layer carried by the layer step's launch: the same results as the
    layer step alone followed by prr_predict."""
    w = wl.Workload("carry_ls", 2, 8, 2, 128, 16384, 16, 32, "bf16", seed=13)
    inp = wl.make_inputs(w, "cuda")
    dkv = device_kv(inp)
    meta = bd.build_meta(dkv, w.block)
    rng = np.random.default_rng(8)
    P = sets_to_device(_random_p(w, rng, [32, 20]), 32)
    B, H, N = w.batch, w.num_kv_heads, bd.max_blocks(dkv, w.block)
    other = torch.from_numpy(rng.standard_normal((B, H, N))).cuda()
    lv0 = torch.from_numpy(rng.standard_normal((B, H, N))).cuda()
    tr0 = torch.from_numpy(rng.standard_normal((B, H, N))).cuda()
    live0 = torch.full((B, H), N // 2, dtype=torch.int32, device="cuda")

    def run(carry):
        lv, tr, live = lv0.clone(), tr0.clone(), live0.clone()
        Pn = bd.BlockSet.empty(B, H, 24)
        args = bd.PredictArgs(other, dkv.seq_len, w.block, 0.6, 0.3, 0.5, 24, lv, tr, live, Pn)
        st = bd.AttnState.empty(B, w.num_q_heads, w.head_dim)
        out = torch.empty_like(st.acc)
        sc = torch.zeros((B, H, N), dtype=torch.float64, device="cuda")
        A, M = bd.BlockSet.empty(B, H, w.topk), bd.BlockSet.empty(B, H, w.topk)
        bd.layer_step(inp.q[0], dkv, meta, w.block, w.topk, P, w.scale, sc, A, M, st, out=out,
                      pred=args if carry else None)
        if not carry:
            bd.predict(other, dkv.seq_len, w.block, 0.6, 0.3, 0.5, 24, lv, tr, live, P_next=Pn)
        torch.cuda.synchronize()
        return sc, A.lists(), M.lists(), st, out, lv, tr, live, Pn.lists()

    a, b = run(True), run(False)
    assert a[1] == b[1] and a[2] == b[2] and a[8] == b[8]
    for x, y in ((a[0], b[0]), (a[3].acc, b[3].acc), (a[3].l, b[3].l), (a[3].m, b[3].m), (a[4], b[4]), (a[5], b[5]),
                 (a[6], b[6]), (a[7], b[7])):
        assert torch.equal(x, y)


def test_layer_step_three_stage_mean_scoring_carrying_a_predictor():
    """The three in-launch ranking stages with block-mean scoring and another layer's predictor step in
    the same launch (32768 blocks, K = 256): scores, A, M, the predictor's state and P_next equal the
    separate calls' bit for bit, and the state theirs within the float32 tolerance (it merges the
    partial states in another grouping)."""
    w = wl.Workload("three_mean_pred", 1, 8, 2, 128, 32768 * 16, 16, 256, "bf16", seed=77)
    inp = wl.make_inputs(w, "cuda")
    dkv = device_kv(inp)
    means = bd.build_mean_meta(dkv, w.block)
    rng = np.random.default_rng(12)
    Pd = sets_to_device(_random_p(w, rng, [256, 100]), 256)
    B, H, N = w.batch, w.num_kv_heads, bd.max_blocks(dkv, w.block)
    other = torch.from_numpy(rng.standard_normal((B, H, N))).cuda()
    lv0 = torch.from_numpy(rng.standard_normal((B, H, N))).cuda()
    tr0 = torch.from_numpy(rng.standard_normal((B, H, N))).cuda()
    live0 = torch.full((B, H), N - 300, dtype=torch.int32, device="cuda")
    q = inp.q[0]

    lv, tr, live = lv0.clone(), tr0.clone(), live0.clone()
    Pn = bd.BlockSet.empty(B, H, 64)
    args = bd.PredictArgs(other, dkv.seq_len, w.block, 0.6, 0.3, 0.5, 64, lv, tr, live, Pn,
                          ws=bd.predict_workspace_for(B, H, N, 64))
    st = bd.AttnState.empty(B, w.num_q_heads, w.head_dim)
    out = torch.empty_like(st.acc)
    sc = torch.zeros((B, H, N), dtype=torch.float64, device="cuda")
    A, M = bd.BlockSet.empty(B, H, w.topk), bd.BlockSet.empty(B, H, w.topk)
    bd.layer_step(q, dkv, means, w.block, w.topk, Pd, w.scale, sc, A, M, st, out=out, mode="mean", pred=args)

    lv2, tr2, live2 = lv0.clone(), tr0.clone(), live0.clone()
    scores, A2, M2 = bd.select(q, dkv, means, w.block, w.topk, P=Pd, mode="mean")
    ref = bd.spec_attn(q, dkv, w.block, Pd, w.scale)
    bd.repair(q, dkv, w.block, M2, w.scale, ref)
    Pn2 = bd.predict(other, dkv.seq_len, w.block, 0.6, 0.3, 0.5, 64, lv2, tr2, live2,
                     ws=bd.predict_workspace_for(B, H, N, 64))
    torch.cuda.synchronize()
    assert torch.equal(sc, scores) and A.lists() == A2.lists() and M.lists() == M2.lists()
    assert Pn.lists() == Pn2.lists()
    assert torch.equal(lv, lv2) and torch.equal(tr, tr2) and torch.equal(live, live2)
    acc, l, m = (t.double().cpu().numpy() for t in (st.acc, st.l, st.m))
    racc, rl, rm = (t.double().cpu().numpy() for t in (ref.acc, ref.l, ref.m))
    assert np.all(rl > 0)
    assert np.all(np.abs(l - rl) <= 1e-4 * rl)
    assert np.all(np.abs(m - rm) <= 1e-4 * np.maximum(1.0, np.abs(rm)))
    assert np.max(np.abs(acc / l[..., None] - racc / rl[..., None])) <= 5e-3
