"""GPU parity of mean-pooled block selection (the block summarised by its mean key, one of the two
summaries the pages name for selection) against the oracle: the fp32 block means bit for bit, the fp64
scores bit for bit, A and M exactly; the fused selection + speculative launch in this mode against the
separate calls.  Sizes span several scoring workgroups (256 blocks each) with a ragged tail, the
fused launch's single-, two- and three-stage top-K, and sequences of one token and of none."""
import numpy as np
import pytest
import torch

from _gpu import assert_heads, device_kv, require_gpu, sets_to_device
from _util import oracle_view
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


CASES = [
    # name, B, Hq, Hkv, d, block, lens, dtype, topk, zero-length sequence index (or None)
    ("bf16_d128_s16_ragged", 2, 8, 2, 128, 16, [20811, 9000], "bf16", 64, None),
    ("f32_d64_s64", 1, 4, 1, 64, 64, [33000], "f32", 40, None),
    ("bf16_d64_s32_short", 3, 8, 1, 64, 32, [4097, 1, 600], "bf16", 16, 2),
    # 2500 blocks: the fused launch ranks per-workgroup candidates (two-stage top-K), K above the 256
    # blocks of one scoring workgroup
    ("bf16_d128_s16_two_stage", 1, 8, 2, 128, 16, [40000], "bf16", 300, None),
    ("fp8_d128_s32", 2, 8, 2, 128, 32, [9000, 4100], "fp8", 32, None),
    # 8192 blocks at K = 600: more candidate slots than one ranking holds, so groups of parts rank
    # their candidates, inside the fused launch (three-stage top-K)
    ("bf16_d64_s16_three_stage", 1, 4, 1, 64, 16, [131072], "bf16", 600, None),
    # 32768 blocks at K = 400: groups of 10 parts (4000 slots) and a ranking of 7 x 400, both at 16
    # candidate slots per thread, inside the launch
    ("bf16_d128_s16_three_stage_k400", 1, 4, 1, 128, 16, [1 << 19], "bf16", 400, None),
]


def _setup(case):
    name, B, Hq, Hkv, d, S, lens, dt, k, zero = case
    w = wl.Workload(name, B, Hq, Hkv, d, max(lens), S, k, dt, seed=500 + S, seq_lens=lens)
    inp = wl.make_inputs(w, "cuda")
    if zero is not None:
        inp.seq_len[zero] = 0
    q, kv = oracle_view(inp)
    return w, inp, q[0], kv


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mean_meta_scores_and_sets(case):
    w, inp, q, kv = _setup(case)
    dkv = device_kv(inp)
    meta = bd.build_mean_meta(dkv, w.block)
    assert meta.dtype == torch.float32 and meta.shape[-1] == bd.meta_stride(dkv, w.block)
    omean = orc.build_mean_meta(kv, w.block, w.num_kv_heads)
    gm = meta.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            nb = omean[b][h].shape[0]
            assert np.array_equal(gm[b, h, :, :nb].T.astype(np.float64), omean[b][h]), (b, h)

    osc, oA, _ = orc.select_mean(q, omean, w.group, w.topk)
    rng = np.random.default_rng(w.seed)
    P = [[np.sort(rng.choice(max(omean[b][h].shape[0], 1), size=min(w.topk, omean[b][h].shape[0]),
                             replace=False)) if omean[b][h].shape[0] else np.zeros(0, dtype=np.int64)
          for h in range(w.num_kv_heads)] for b in range(w.batch)]
    Pd = sets_to_device(P, w.topk)
    scores, A, M = bd.select(inp.q[0], dkv, meta, w.block, w.topk, P=Pd, mode="mean")
    sc = scores.cpu().numpy()
    Al, Ml = A.lists(), M.lists()
    for b in range(w.batch):
        for h in range(w.num_kv_heads):
            nb = omean[b][h].shape[0]
            assert np.array_equal(sc[b, h, :nb], osc[b][h]), (b, h)
            assert Al[b][h] == list(oA[b][h]), (b, h)
            assert Ml[b][h] == list(orc.set_minus(oA[b][h], P[b][h])), (b, h)

    # selection + speculative pass in one call, this mode: the same scores, sets and state as the
    # separate calls
    fs, fA, fM, fstate = bd.select_spec(inp.q[0], dkv, meta, w.block, w.topk, Pd, w.scale, mode="mean")
    state = bd.spec_attn(inp.q[0], dkv, w.block, Pd, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(fs, scores)
    assert fA.lists() == Al and fM.lists() == Ml
    for x, y in ((fstate.acc, state.acc), (fstate.l, state.l), (fstate.m, state.m)):
        assert torch.equal(x, y)
    spec_ref = orc.spec_states(q, kv, w.block, P, w.scale)
    assert_heads(fstate, spec_ref, "spec (mean mode)")


def test_quest_and_mean_metadata_are_not_interchangeable():
    """Selection reads the metadata its mode names: the same scores from the same inputs in each mode
    agree with their own oracle and differ from each other."""
    case = CASES[0]
    w, inp, q, kv = _setup(case)
    dkv = device_kv(inp)
    s_q, _, _ = bd.select(inp.q[0], dkv, bd.build_meta(dkv, w.block), w.block, w.topk)
    s_m, _, _ = bd.select(inp.q[0], dkv, bd.build_mean_meta(dkv, w.block), w.block, w.topk, mode="mean")
    oq, _, _ = orc.select(q, orc.build_meta(kv, w.block, w.num_kv_heads), w.group, w.topk)
    nb = oq[0][0].shape[0]
    assert np.array_equal(s_q[0, 0, :nb].cpu().numpy(), oq[0][0])
    assert not np.array_equal(s_q[0, 0, :nb].cpu().numpy(), s_m[0, 0, :nb].cpu().numpy())
