"""The predictor over long rows: with a workspace, rows of more than 2048 blocks are updated by 512-block
parts and P_next is ranked from the parts' candidates (through groups of parts when the candidate slots
outnumber one ranking's).  Against the one-workgroup-per-row path and the
oracle, step by step (births at the first step, several steps, ragged lengths, budgets below and above
one part's 512 blocks): level, trend, live and P_next bit for bit."""
import numpy as np
import pytest
import torch

from _gpu import require_gpu
from block_sparse_attention_quest_amd import binding as bd
from oracle import prr_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


CASES = [
    # name, B, Hkv, block, lens, budget
    ("n8192_k128", 2, 2, 16, [131072, 100000], 128),
    ("n3500_k600", 1, 2, 32, [112000], 600),
    ("n3000_k64_ragged", 3, 1, 16, [48000, 2000, 33000], 64),
    # more candidate slots than one ranking holds: groups of parts in between (three stages)
    ("n32768_k256_three", 1, 2, 16, [524288], 256),
    ("n16384_k300_three_ragged", 2, 1, 16, [262144, 150000], 300),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_two_stage_predictor_matches_single_workgroup_and_oracle(case):
    name, B, H, block, lens, budget = case
    nmax = -(-max(lens) // block)
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    ws = bd.predict_workspace_for(B, H, nmax, budget)
    assert ws is not None
    rng = np.random.default_rng(len(name))
    state = {k: (torch.zeros((B, H, nmax), dtype=torch.float64, device="cuda"),
                 torch.zeros((B, H, nmax), dtype=torch.float64, device="cuda"),
                 torch.zeros((B, H), dtype=torch.int32, device="cuda")) for k in ("two", "one")}
    ost = {(b, h): (np.zeros(0), np.zeros(0), 0) for b in range(B) for h in range(H)}
    alpha, beta, gamma = 0.6, 0.3, 0.5
    for step in range(4):
        # scores with repeated values, so ties are broken by index across part boundaries
        s = np.round(rng.lognormal(0.0, 1.0, size=(B, H, nmax)), 2)
        scores = torch.from_numpy(s).cuda()
        Pt = bd.predict(scores, seq_len, block, alpha, beta, gamma, budget, *state["two"], ws=ws)
        Po = bd.predict(scores, seq_len, block, alpha, beta, gamma, budget, *state["one"])
        torch.cuda.synchronize()
        for a, b in zip(state["two"], state["one"]):
            assert torch.equal(a, b), step
        assert Pt.lists() == Po.lists(), step
        lv_d = state["two"][0].cpu().numpy()
        tr_d = state["two"][1].cpu().numpy()
        for b in range(B):
            nb = -(-lens[b] // block)
            for h in range(H):
                lv, tr, live = ost[(b, h)]
                lv, tr, live, P = orc.predict_step(lv, tr, live, s[b, h, :nb], alpha, beta, gamma, budget)
                assert np.array_equal(lv_d[b, h, :nb], lv) and np.array_equal(tr_d[b, h, :nb], tr), (step, b, h)
                assert Pt.lists()[b][h] == list(P), (step, b, h)
                ost[(b, h)] = (lv, tr, live)
        assert state["two"][2].cpu().tolist() == [[-(-x // block)] * H for x in lens]
