"""GPU parity with heavy exact ties at full row lengths.  Every block of a row copies the keys of one of a
few source blocks, so the Quest scores take a few values, each shared by dozens to hundreds of blocks, and
the top-K boundary falls inside a group of equal scores.  Every ranking path must then take the tied blocks
with the smaller indices, as the oracle's brute-force ranking does: one top-K workgroup per row, the
part-parallel stages of prr_select, the fused launch's two and three stages (prr_select_spec and
prr_layer_step), and the predictor's top-|P|, whose first step (every block new) predicts each block's
score.  A, M and P on every unit against the oracle.
"""
import numpy as np
import pytest
import torch

from _gpu import device_kv, require_gpu, sets_to_device, unit_meta, unit_view
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


def _say(msg):
    print(f"[ties at scale] {msg}", flush=True)


# (id, blocks per row, K, distinct source blocks): 2048 blocks in 37 groups of about 55 (the boundary
# inside the second group), 8192 in 53 groups of about 155 and 40000 in 61 groups of about 656 (the
# boundary inside the top group; 40000 blocks rank in three stages)
CASES = [("2048_k64", 2048, 64, 37), ("8192_k128", 8192, 128, 53), ("40000_k256", 40000, 256, 61)]


@pytest.mark.parametrize("name,nb,topk,nsrc", CASES, ids=[c[0] for c in CASES])
def test_tied_rows_rank_by_index_on_every_path(name, nb, topk, nsrc):
    w = wl.Workload(f"ties_{name}", 2, 8, 2, 64, nb * 16, 16, topk, "bf16", seed=70 + nsrc)
    _say(f"{name}: inputs ({nb} blocks, K = {topk}, {nsrc} distinct blocks)")
    inp = wl.make_inputs(w, "cuda")
    # block p of every row (one page at block 16) takes the keys of block p mod nsrc of its row
    for b in range(w.batch):
        pt = inp.page_table[b, :nb].long()
        src = pt[torch.arange(nb, device=pt.device) % nsrc]
        inp.k_cache[pt] = inp.k_cache[src].clone()
    kv = device_kv(inp)
    meta = bd.build_meta(kv, w.block)
    B, H = w.batch, w.num_kv_heads
    # the oracle's scores and A on every unit
    ref_s, ref_a = {}, {}
    for b in range(B):
        for h in range(H):
            q, ukv = unit_view(inp, b, h)
            mn, mx = unit_meta(ukv, w.block)
            s = orc.quest_scores(orc.representative_query(q, 0, 0, w.group), mn, mx)
            assert len(np.unique(s)) <= nsrc
            ref_s[(b, h)] = s
            ref_a[(b, h)] = orc.topk_blocks(s, topk)
    P = [[list(wl.make_spec_set(w, ref_a[(b, h)], nb, topk // 2, topk // 4, salt=b * H + h)) for h in range(H)]
         for b in range(B)]
    Pd = sets_to_device(P, topk)

    def check(what, scores, A, M=None):
        got_a = A.lists()
        got_m = M.lists() if M is not None else None
        for b in range(B):
            for h in range(H):
                assert np.array_equal(scores[b, h, :nb].cpu().numpy(), ref_s[(b, h)]), (what, b, h)
                assert got_a[b][h] == list(ref_a[(b, h)]), (what, b, h)
                if got_m is not None:
                    assert got_m[b][h] == list(orc.set_minus(ref_a[(b, h)], P[b][h])), (what, b, h)

    if nb <= 32768:
        _say(f"{name}: prr_select, one top-K workgroup per row")
        s1, A1, M1 = bd.select(inp.q[0], kv, meta, w.block, topk, P=Pd, staged=False)
        torch.cuda.synchronize()
        check("select one workgroup", s1, A1, M1)
    _say(f"{name}: prr_select with its workspace")
    s2, A2, M2 = bd.select(inp.q[0], kv, meta, w.block, topk, P=Pd)
    torch.cuda.synchronize()
    check("select", s2, A2, M2)
    _say(f"{name}: prr_select_spec")
    s3, A3, M3, _ = bd.select_spec(inp.q[0], kv, meta, w.block, topk, Pd, w.scale)
    torch.cuda.synchronize()
    check("select_spec", s3, A3, M3)
    _say(f"{name}: prr_layer_step")
    s4 = torch.zeros_like(s3)
    A4, M4 = bd.BlockSet.empty(B, H, topk), bd.BlockSet.empty(B, H, topk)
    st = bd.AttnState.empty(B, w.num_q_heads, w.head_dim)
    bd.layer_step(inp.q[0], kv, meta, w.block, topk, Pd, w.scale, s4, A4, M4, st)
    torch.cuda.synchronize()
    check("layer_step", s4, A4, M4)
    # the predictor's first step: every block is new (level = IS, trend = 0), so the prediction is the
    # score itself and P_next = the top-|P| of the tied scores
    _say(f"{name}: prr_predict")
    budget = topk // 2
    level = torch.zeros((B, H, w.max_blocks), dtype=torch.float64, device="cuda")
    trend = torch.zeros_like(level)
    live = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    ws = bd.predict_workspace_for(B, H, w.max_blocks, budget)
    Pn = bd.predict(s2, kv.seq_len, w.block, 0.6, 0.3, 0.5, budget, level, trend, live, ws=ws)
    torch.cuda.synchronize()
    got_p = Pn.lists()
    for b in range(B):
        for h in range(H):
            _, _, _, p_ref = orc.predict_step(np.zeros(0), np.zeros(0), 0, ref_s[(b, h)], 0.6, 0.3, 0.5, budget)
            assert got_p[b][h] == list(p_ref), (b, h)
