"""Page work lists (the `pages` member of prr_block_set): written by the calls that produce a set, read by the
attention passes over it ([paper] §4.3: the repair kernel reads the missed blocks' tiles; the predictor
produces P a step early, [paper] §4.1).

Each writer's list is checked slot by slot against its definition, computed on the host from the set it
wrote and the page table: slot e * ppb + s of a unit is the physical page of page s of the set's block e,
or -1 where that page held no token (the comparison is exact).  The writers are: the separate top-K
(prr_select), the top-K inside the selection + speculation launch (one- and two-stage), the layer step's
top-K (one launch, and its three-stage fallback), the predictor on its own (one workgroup per row, rows
in parts, three stages) and the predictor carried by a selection launch.

The readers (speculative pass, repair, the selection + speculation launch and the layer step) give
bit-identical results with and without a list: the list only says where the pages are.  A list written
before the sequences grew, with the pages that held no token then mapped elsewhere afterwards, still
gives the results of a list-free call: such slots are -1 and are looked up when read.
"""
import numpy as np
import pytest
import torch

from _gpu import device_kv, require_gpu, sets_to_device
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


def expected_list(idx, cnt, page_table, seq_len, block):
    """Host definition of a set's page list: [B][H][cap * ppb], slots past count * ppb left at -2."""
    B, H, cap = idx.shape
    ppb = block // wl.PAGE_SIZE
    out = np.full((B, H, cap * ppb), -2, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for e in range(int(cnt[b, h])):
                for s in range(ppb):
                    lp = int(idx[b, h, e]) * ppb + s
                    ok = lp < page_table.shape[1] and lp * wl.PAGE_SIZE < int(seq_len[b])
                    out[b, h, e * ppb + s] = int(page_table[b, lp]) if ok else -1
    return out


def assert_list(S: bd.BlockSet, page_table, seq_len, block, what):
    idx, cnt = S.idx.cpu().numpy(), S.count.cpu().numpy()
    ref = expected_list(idx, cnt, page_table.cpu().numpy(), seq_len.cpu().numpy(), block)
    got = S.pages.cpu().numpy().astype(np.int64)
    mask = ref != -2
    assert mask.any() or cnt.sum() == 0, what
    bad = np.argwhere(mask & (got != ref))
    assert bad.size == 0, f"{what}: {len(bad)} slots differ, first {bad[:4].tolist()}"


def listed(S: bd.BlockSet, block: int) -> bd.BlockSet:
    """A copy of S with a page list (filled by -1: not yet written)."""
    B, H, cap = S.idx.shape
    out = bd.BlockSet.empty(B, H, cap, S.idx.device, block)
    out.idx.copy_(S.idx)
    out.count.copy_(S.count)
    return out


def _case(dtype="bf16", context=4000, batch=2, block=64, topk=16, seed=7, hkv=2, hq=8, d=128):
    """Ragged lengths that end inside a page (so some pages of the last blocks hold no token)."""
    lens = tuple(max(1, context - 37 * b - 3) for b in range(batch))
    w = wl.Workload("lists", batch, hq, hkv, d, context, block, topk, dtype, seed=seed, seq_lens=lens)
    inp = wl.make_inputs(w, "cuda")
    return w, inp, device_kv(inp)


def _random_p(w, seed, n):
    rng = np.random.default_rng(seed)
    return [[sorted(rng.permutation(w.blocks_of(b))[:min(n, w.blocks_of(b))].tolist())
             for _ in range(w.num_kv_heads)] for b in range(w.batch)]


@pytest.mark.parametrize("block", [16, 64, 256])
def test_select_writes_m_list(block):
    w, inp, kv = _case(block=block, context=5000, topk=12)
    meta = bd.build_meta(kv, w.block)
    P = sets_to_device(_random_p(w, 1, 8), 8)
    B, H = w.batch, w.num_kv_heads
    A = bd.BlockSet.empty(B, H, w.topk)
    M = bd.BlockSet.empty(B, H, w.topk, "cuda", w.block)
    bd.select(inp.q[0], kv, meta, w.block, w.topk, P=P, A=A, M=M)
    torch.cuda.synchronize()
    assert_list(M, inp.page_table, inp.seq_len, w.block, f"select M list, block {block}")


@pytest.mark.parametrize("context,topk", [(4000, 16), (70000, 40)])   # one-stage / two-stage top-K
def test_select_spec_lists_and_results(context, topk):
    """M's list from the fused launch's top-K; P's list read by its speculative workgroups."""
    w, inp, kv = _case(context=context, topk=topk, batch=1, hkv=4, hq=16)
    meta = bd.build_meta(kv, w.block)
    P0 = sets_to_device(_random_p(w, 2, topk), topk)
    B, H = w.batch, w.num_kv_heads
    # P0 with its list as the predictor would write it (the definition, on the host)
    Pl = listed(P0, w.block)
    ref = expected_list(P0.idx.cpu().numpy(), P0.count.cpu().numpy(), inp.page_table.cpu().numpy(),
                        inp.seq_len.cpu().numpy(), w.block)
    Pl.pages.copy_(torch.from_numpy(np.where(ref == -2, -1, ref).astype(np.int32)).cuda())
    outs = []
    for P, M in ((P0, bd.BlockSet.empty(B, H, topk)), (Pl, bd.BlockSet.empty(B, H, topk, "cuda", w.block))):
        scores, A, M, st = bd.select_spec(inp.q[0], kv, meta, w.block, topk, P, w.scale, M=M)
        torch.cuda.synchronize()
        outs.append((scores, A.lists(), M.lists(), st))
    assert torch.equal(outs[0][0], outs[1][0]) and outs[0][1] == outs[1][1] and outs[0][2] == outs[1][2]
    for name in ("acc", "l", "m"):
        assert torch.equal(getattr(outs[0][3], name), getattr(outs[1][3], name)), name
    assert_list(M, inp.page_table, inp.seq_len, w.block, "select_spec M list")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_spec_and_repair_read_lists(dtype):
    w, inp, kv = _case(dtype=dtype, context=6000, topk=24)
    B, H = w.batch, w.num_kv_heads
    S = sets_to_device(_random_p(w, 3, 24), 24)
    L = listed(S, w.block)
    ref = expected_list(S.idx.cpu().numpy(), S.count.cpu().numpy(), inp.page_table.cpu().numpy(),
                        inp.seq_len.cpu().numpy(), w.block)
    L.pages.copy_(torch.from_numpy(np.where(ref == -2, -1, ref).astype(np.int32)).cuda())
    a = bd.spec_attn(inp.q[0], kv, w.block, S, w.scale)
    b = bd.spec_attn(inp.q[0], kv, w.block, L, w.scale)
    base = bd.spec_attn(inp.q[0], kv, w.block, sets_to_device(_random_p(w, 4, 8), 8), w.scale)
    ra, rb = base.clone(), base.clone()
    oa, ob = torch.empty_like(ra.acc), torch.empty_like(rb.acc)
    bd.repair(inp.q[0], kv, w.block, S, w.scale, ra, out=oa)
    bd.repair(inp.q[0], kv, w.block, L, w.scale, rb, out=ob)
    torch.cuda.synchronize()
    for name in ("acc", "l", "m"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
        assert torch.equal(getattr(ra, name), getattr(rb, name)), name
    assert torch.equal(oa, ob)


def test_stale_list_after_growth_reads_the_new_pages():
    """P's list is written at one length; the sequences then grow into pages that held no token before,
    and those pages are mapped to other physical pages (as an allocator would map them at first write).
    The list's -1 slots are looked up when read: the pass equals a list-free one on the new mapping."""
    w, inp, kv = _case(context=3000, block=64, topk=64, batch=2)
    B, H = w.batch, w.num_kv_heads
    lens0 = inp.seq_len.clone()
    nb = [w.blocks_of(b) for b in range(B)]
    # P = every block of each sequence (its last, partly filled block included), with its list at lens0
    P = sets_to_device([[list(range(nb[b]))] * H for b in range(B)], max(nb))
    L = listed(P, w.block)
    ref = expected_list(P.idx.cpu().numpy(), P.count.cpu().numpy(), inp.page_table.cpu().numpy(),
                        lens0.cpu().numpy(), w.block)
    L.pages.copy_(torch.from_numpy(np.where(ref == -2, -1, ref).astype(np.int32)).cuda())
    assert (ref == -1).any()   # some pages of the last blocks held no token
    # grow every sequence to the end of its last block and remap the pages that were empty at lens0
    ppb = w.block // wl.PAGE_SIZE
    pt = inp.page_table.cpu().numpy().copy()
    rng = np.random.default_rng(5)
    for b in range(B):
        first_empty = (int(lens0[b]) + wl.PAGE_SIZE - 1) // wl.PAGE_SIZE
        for lp in range(first_empty, nb[b] * ppb):
            pt[b, lp] = int(rng.integers(0, w.num_pages))
    inp.page_table.copy_(torch.from_numpy(pt).to(inp.page_table.device))
    inp.seq_len.copy_(torch.tensor([nb[b] * w.block for b in range(B)], dtype=torch.int32))
    kv2 = device_kv(inp)
    a = bd.spec_attn(inp.q[0], kv2, w.block, P, w.scale)
    b = bd.spec_attn(inp.q[0], kv2, w.block, L, w.scale)
    torch.cuda.synchronize()
    for name in ("acc", "l", "m"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


@pytest.mark.parametrize("dtype,context,topk", [("bf16", 4000, 16), ("fp8", 4000, 16), ("bf16", 70000, 40),
                                                ("bf16", 32768 * 64, 256)])
def test_layer_step_lists(dtype, context, topk):
    """One launch (bf16, fp8; one- and two-stage top-K) and the three-stage fallback (32768 blocks at
    K = 256, batch 1, one kv head): M's list as defined, results bitwise those of a list-free step."""
    if context > 100000:
        w, inp, kv = _case(dtype=dtype, context=context, topk=topk, batch=1, hkv=1, hq=4, block=64)
    else:
        w, inp, kv = _case(dtype=dtype, context=context, topk=topk)
    meta = bd.build_meta(kv, w.block)
    B, H = w.batch, w.num_kv_heads
    P0 = sets_to_device(_random_p(w, 6, topk), topk)
    Pl = listed(P0, w.block)
    ref = expected_list(P0.idx.cpu().numpy(), P0.count.cpu().numpy(), inp.page_table.cpu().numpy(),
                        inp.seq_len.cpu().numpy(), w.block)
    Pl.pages.copy_(torch.from_numpy(np.where(ref == -2, -1, ref).astype(np.int32)).cuda())
    res = []
    for P, lb in ((P0, 0), (Pl, w.block)):
        scores = torch.zeros((B, H, bd.max_blocks(kv, w.block)), dtype=torch.float64, device="cuda")
        A, M = bd.BlockSet.empty(B, H, topk), bd.BlockSet.empty(B, H, topk, "cuda", lb)
        st = bd.AttnState.empty(B, w.num_q_heads, w.head_dim)
        out = torch.empty_like(st.acc)
        bd.layer_step(inp.q[0], kv, meta, w.block, topk, P, w.scale, scores, A, M, st, out=out)
        torch.cuda.synchronize()
        res.append((scores, A.lists(), M, st, out))
    assert torch.equal(res[0][0], res[1][0]) and res[0][1] == res[1][1] and res[0][2].lists() == res[1][2].lists()
    for name in ("acc", "l", "m"):
        assert torch.equal(getattr(res[0][3], name), getattr(res[1][3], name)), name
    assert torch.equal(res[0][4], res[1][4])
    assert_list(res[1][2], inp.page_table, inp.seq_len, w.block, f"layer step M list ({dtype}, {context})")


def _predict_case(nmax_blocks, block, batch, hkv, seed):
    """Scores and lengths for a predictor step, and a cache description whose page table the list maps
    through (the predictor reads no K/V: one page of it is enough)."""
    rng = np.random.default_rng(seed)
    ppb = block // wl.PAGE_SIZE
    max_pages = nmax_blocks * ppb
    lens = rng.integers(nmax_blocks * block // 2, nmax_blocks * block + 1, size=batch).astype(np.int32)
    pt = rng.integers(0, 1 << 20, size=(batch, max_pages)).astype(np.int32)
    k = torch.zeros((1, hkv, wl.PAGE_SIZE, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((1, hkv, 128, wl.PAGE_SIZE), dtype=torch.bfloat16, device="cuda")
    seq_len = torch.from_numpy(lens).cuda()
    kv = bd.KVCache(k, v, torch.from_numpy(pt).cuda(), seq_len)
    scores = torch.from_numpy(rng.standard_normal((batch, hkv, nmax_blocks))).cuda()
    return kv, scores, seq_len


@pytest.mark.parametrize("nmax,budget,use_ws", [(1000, 48, False), (2500, 64, True), (32768, 400, True),
                                                (2048, 2048, False)])
def test_predict_writes_p_list(nmax, budget, use_ws):
    """One workgroup per row, rows in parts, three stages; and a budget covering whole rows (the rows'
    last blocks, partly filled, get -1 slots)."""
    block = 16 if nmax > 2048 else 64
    B, H = 2, 2
    kv, scores, seq_len = _predict_case(nmax, block, B, H, seed=nmax + budget)
    lv, tr = torch.zeros_like(scores), torch.zeros_like(scores)
    live = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    ws = bd.predict_workspace_for(B, H, nmax, budget, "cuda") if use_ws else None
    Pn = bd.BlockSet.empty(B, H, budget, "cuda", block)
    Pr = bd.BlockSet.empty(B, H, budget, "cuda")
    lv2, tr2, live2 = lv.clone(), tr.clone(), live.clone()
    bd.predict(scores, seq_len, block, 0.6, 0.3, 0.5, budget, lv, tr, live, P_next=Pn, ws=ws, kv=kv)
    bd.predict(scores, seq_len, block, 0.6, 0.3, 0.5, budget, lv2, tr2, live2, P_next=Pr, ws=ws)
    torch.cuda.synchronize()
    assert Pn.lists() == Pr.lists() and torch.equal(lv, lv2) and torch.equal(tr, tr2)
    assert_list(Pn, kv.page_table, seq_len, block, f"predict P list ({nmax}, {budget})")


def test_carried_predictor_writes_p_list():
    w, inp, kv = _case(context=4000, topk=16)
    meta = bd.build_meta(kv, w.block)
    B, H = w.batch, w.num_kv_heads
    nmax = bd.max_blocks(kv, w.block)
    rng = np.random.default_rng(11)
    other = torch.from_numpy(rng.standard_normal((B, H, nmax))).cuda()
    lv, tr = torch.zeros_like(other), torch.zeros_like(other)
    live = torch.zeros((B, H), dtype=torch.int32, device="cuda")
    Pn = bd.BlockSet.empty(B, H, 20, "cuda", w.block)
    args = bd.PredictArgs(other, kv.seq_len, w.block, 0.6, 0.3, 0.5, 20, lv, tr, live, Pn, None, kv)
    P = sets_to_device(_random_p(w, 9, 16), 16)
    for call in ("select_spec", "layer_step"):
        Pn.pages.fill_(-7)
        lv.zero_(); tr.zero_(); live.zero_()
        A, M = bd.BlockSet.empty(B, H, 16), bd.BlockSet.empty(B, H, 16)
        scores = torch.zeros((B, H, nmax), dtype=torch.float64, device="cuda")
        st = bd.AttnState.empty(B, w.num_q_heads, w.head_dim)
        if call == "select_spec":
            bd.select_spec(inp.q[0], kv, meta, w.block, 16, P, w.scale, scores=scores, A=A, M=M, out=st, pred=args)
        else:
            bd.layer_step(inp.q[0], kv, meta, w.block, 16, P, w.scale, scores, A, M, st, pred=args)
        torch.cuda.synchronize()
        assert_list(Pn, inp.page_table, inp.seq_len, w.block, f"carried predictor P list ({call})")
