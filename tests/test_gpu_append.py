"""Decode-loop continuity on the GPU: prr_append against the definition of the paged layout and against
metadata rebuilt from scratch (device and oracle), and a decode trajectory that appends one token per
sequence before every layer step, checked unit by unit against the oracle (blocks are born mid-run)."""
import numpy as np
import pytest
import torch

from _gpu import assert_state, device_kv, require_gpu, unit_meta, unit_view
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl
from block_sparse_attention_quest_amd.layer_step import PRRLayer
from oracle import prr_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


def _expected_append(k, v, page_table, seq_len, k_new, v_new):
    """The layout's definition on host tensors: token t = seq_len[b] of sequence b lives in physical page
    page_table[b][t // 16], slot t % 16 (K token-major, V channel-major); then seq_len[b] = t + 1.  A
    sequence whose cache is full is left as it is."""
    max_tokens = page_table.shape[1] * wl.PAGE_SIZE
    for b in range(page_table.shape[0]):
        t = int(seq_len[b])
        if t >= max_tokens:
            continue
        ph = int(page_table[b, t // wl.PAGE_SIZE])
        k[ph, :, t % wl.PAGE_SIZE, :] = k_new[b]
        v[ph, :, :, t % wl.PAGE_SIZE] = v_new[b]
        seq_len[b] = t + 1


def _host_inputs(inp, k, v, seq_len):
    return wl.Inputs(inp.w, inp.q.cpu(), k, v, inp.page_table.cpu(), seq_len)


APPEND_CASES = [
    # name, B, Hq, Hkv, d, block, lens, dtype, appended tokens
    ("bf16_d128_s32", 2, 8, 2, 128, 32, [1000, 1023], "bf16", 70),
    ("bf16_d64_s64", 2, 4, 1, 64, 64, [640, 17], "bf16", 50),
    ("f32_d64_s16", 1, 4, 1, 64, 16, [500], "f32", 40),
    ("fp8_d128_s32", 2, 8, 2, 128, 32, [700, 1023], "fp8", 45),
]


@pytest.mark.parametrize("mode", ["quest", "mean"])
@pytest.mark.parametrize("case", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_append_matches_definition_and_rebuild(case, mode):
    name, B, Hq, Hkv, d, S, lens, dt, n = case
    w = wl.Workload(name, B, Hq, Hkv, d, max(lens), S, 4, dt, seed=300 + n, seq_lens=lens, append_tokens=n)
    inp = wl.make_inputs(w, "cuda")
    dkv = device_kv(inp)
    build = bd.build_meta if mode == "quest" else bd.build_mean_meta
    meta = build(dkv, S)
    k_host, v_host = inp.k_cache.cpu().clone(), inp.v_cache.cpu().clone()
    pt, sl = inp.page_table.cpu(), inp.seq_len.cpu().clone()
    kn, vn = wl.make_append_tokens(w, "cuda")
    for t in range(n):
        bd.append(dkv, S, kn[t], vn[t], meta, mode=mode)
        _expected_append(k_host, v_host, pt, sl, kn[t].cpu(), vn[t].cpu())
    torch.cuda.synchronize()
    assert torch.equal(inp.seq_len.cpu(), sl)
    bits = {"bf16": torch.int16, "f32": torch.int32, "fp8": torch.uint8}[dt]
    assert torch.equal(inp.k_cache.cpu().view(bits), k_host.view(bits))
    assert torch.equal(inp.v_cache.cpu().view(bits), v_host.view(bits))
    # the incrementally kept metadata equals a rebuild, bit for bit, on every existing block
    rebuilt = build(dkv, S)
    gm = wl.to_numpy_bits(meta)
    gr = wl.to_numpy_bits(rebuilt)
    _, okv = _host_kv(w, k_host, v_host, pt, sl)
    if mode == "mean":
        omean = orc.build_mean_meta(okv, S, Hkv)
        for b in range(B):
            nb = -(-int(sl[b]) // S)
            assert np.array_equal(gm[b, ..., :nb], gr[b, ..., :nb]), b
            for h in range(Hkv):
                assert np.array_equal(gm[b, h, :, :nb].T.astype(np.float64), omean[b][h]), (b, h)
        return
    ometa = orc.build_meta(okv, S, Hkv)
    for b in range(B):
        nb = -(-int(sl[b]) // S)
        assert np.array_equal(gm[b, :, :, :, :nb], gr[b, :, :, :, :nb]), b
        up = orc.upcast(gm[b, :, :, :, :nb], w.dtype)
        for h in range(Hkv):
            assert np.array_equal(up[h, :, 0, :].T, ometa[b][h][0]), (b, h)
            assert np.array_equal(up[h, :, 1, :].T, ometa[b][h][1]), (b, h)


def _host_kv(w, k, v, pt, sl):
    q = np.zeros((1, w.batch, w.num_q_heads, w.head_dim))
    return q, orc.make_paged_kv(wl.to_numpy_bits(k), wl.to_numpy_bits(v), wl.to_numpy_bits(pt),
                                wl.to_numpy_bits(sl), w.dtype)


@pytest.mark.parametrize("mode", ["quest", "mean"])
def test_append_to_a_full_cache_changes_nothing(mode):
    # 1024 tokens in blocks of 64: the page table has exactly 64 pages, all full
    w = wl.Workload("full", 2, 4, 1, 64, 1024, 64, 4, "bf16", seed=77)
    inp = wl.make_inputs(w, "cuda")
    dkv = device_kv(inp)
    meta = (bd.build_meta if mode == "quest" else bd.build_mean_meta)(dkv, w.block)
    before = (inp.k_cache.clone(), inp.v_cache.clone(), meta.clone(), inp.seq_len.clone())
    ww = wl.scaled(w, append_tokens=1)
    kn, vn = wl.make_append_tokens(ww, "cuda")
    bd.append(dkv, w.block, kn[0], vn[0], meta, mode=mode)
    torch.cuda.synchronize()
    for a, b in zip((inp.k_cache, inp.v_cache, meta, inp.seq_len), before):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("mode", ["quest", "mean"])
def test_decode_trajectory_with_appends(mode, dtype):
    """Every step appends one token per sequence, then runs the one-stream layer step.  Per unit and
    step: scores, A, M, the predictor state and P^{t+1} bit for bit, the repaired state and output within
    tolerance, all against the oracle on the host copy of the grown cache.  Sequence 1 starts a new
    block mid-run.  Both block summaries: Quest's min/max bound and the mean key."""
    steps = 6
    w = wl.Workload("append_traj", 2, 8, 2, 128, 2000, 32, 8, dtype, seed=31, steps=steps,
                    seq_lens=[2000, 1950], drift_rho=0.9, query_mean_gain=0.64, block_centre_std=0.35,
                    append_tokens=steps)
    inp = wl.make_inputs(w, "cuda")
    dkv = device_kv(inp)
    layer = PRRLayer(dkv, w.num_q_heads, w.block, w.topk, w.topk, ema=w.ema, scale=w.scale, score_mode=mode)
    alpha, beta, gamma = w.ema
    kn, vn = wl.make_append_tokens(w, "cuda")
    k_host, v_host = inp.k_cache.cpu().clone(), inp.v_cache.cpu().clone()
    pt, sl = inp.page_table.cpu(), inp.seq_len.cpu().clone()
    units = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    ost = {u: (np.zeros(0), np.zeros(0), 0, np.zeros(0, dtype=np.int64)) for u in units}
    born = False
    for t in range(steps):
        nb_before = [-(-int(x) // w.block) for x in sl]
        layer.append(kn[t], vn[t])
        _expected_append(k_host, v_host, pt, sl, kn[t].cpu(), vn[t].cpu())
        born |= any(-(-int(x) // w.block) > n for x, n in zip(sl, nb_before))
        P_before = layer.P_cur.lists()
        out = layer.step(inp.q[t])
        torch.cuda.synchronize()
        host = _host_inputs(inp, k_host, v_host, sl)
        scores = layer.scores.cpu().numpy()
        lv_dev, tr_dev = layer.level.cpu().numpy(), layer.trend.cpu().numpy()
        A, M, Pn = layer.A.lists(), layer.M.lists(), layer.P_cur.lists()
        acc, l, m = (x.double().cpu().numpy() for x in (layer.state.acc, layer.state.l, layer.state.m))
        o = out.double().cpu().numpy()
        for (b, h) in units:
            lv, tr, live, P = ost[(b, h)]
            assert sorted(P_before[b][h]) == list(P), (t, b, h)
            q, kv = unit_view(host, b, h, step=t, length=int(sl[b]))
            qbar = orc.representative_query(q, 0, 0, w.group)
            if mode == "quest":
                mn, mx = unit_meta(kv, w.block)
                s = orc.quest_scores(qbar, mn, mx)
            else:
                s = orc.mean_scores(qbar, orc.build_mean_meta(kv, w.block, 1)[0][0])
            a = orc.topk_blocks(s, w.topk)
            nb = s.shape[0]
            assert np.array_equal(scores[b, h, :nb], s), (t, b, h)
            assert A[b][h] == list(a), (t, b, h)
            m_h = orc.set_minus(a, P)
            assert M[b][h] == list(m_h), (t, b, h)
            blocks = sorted(set(P.tolist()) | set(m_h.tolist()))
            for g in range(w.group):
                ref = orc.head_state(q, kv, 0, g, w.group, blocks, w.block, w.scale)
                hq = h * w.group + g
                assert_state(acc[b, hq], l[b, hq], m[b, hq], ref, f"step {t} b={b} h={h} g={g}")
                assert np.max(np.abs(o[b, hq] - ref.out)) <= 5e-3
            lv, tr, live, P = orc.predict_step(lv, tr, live, s, alpha, beta, gamma, w.topk)
            assert np.array_equal(lv_dev[b, h, :nb], lv) and np.array_equal(tr_dev[b, h, :nb], tr), (t, b, h)
            assert Pn[b][h] == list(P), (t, b, h)
            ost[(b, h)] = (lv, tr, live, P)
    assert born, "the trajectory should start a new block"
