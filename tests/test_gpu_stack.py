"""A stack of layers through several decode steps, with each layer's predictor step carried by the next
layer's selection + speculative launch (prr_select_spec_predict), against the same layers run one
step at a time with the predictor on its own: every set, score, predictor state and output bit for bit.
Covers carried predictor rows inside the launch (up to 2048 blocks) and after it (longer rows), fp32
and bf16 caches, both block summaries, appends, and a one-layer stack."""
import numpy as np
import pytest
import torch

from _gpu import device_kv, require_gpu
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl
from block_sparse_attention_quest_amd.layer_step import PRRLayer, PRRStack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


def _workloads(steps):
    common = dict(steps=steps, drift_rho=0.9, query_mean_gain=0.64, block_centre_std=0.35, append_tokens=steps)
    return [
        # (workload, score mode)
        (wl.Workload("l0", 2, 8, 2, 128, 8000, 16, 32, "bf16", seed=41, seq_lens=[8000, 7001],
                     ema=(0.6, 0.3, 0.5), **common), "quest"),
        (wl.Workload("l1", 1, 8, 2, 128, 40000, 16, 64, "bf16", seed=42, ema=(0.8, 0.1, 0.25), **common),
         "quest"),   # 2500 blocks: its carried predictor runs after the next launch
        (wl.Workload("l2", 2, 4, 1, 64, 3000, 32, 16, "bf16", seed=43, ema=(0.4, 0.5, 0.0), **common), "mean"),
        (wl.Workload("l3", 1, 4, 1, 64, 2000, 16, 8, "f32", seed=44, ema=(0.2, 0.2, 0.75), **common), "quest"),
    ]


def _build(specs):
    layers, inputs, apps = [], [], []
    for w, mode in specs:
        inp = wl.make_inputs(w, "cuda")
        kv = device_kv(inp)
        layers.append(PRRLayer(kv, w.num_q_heads, w.block, w.topk, w.topk, ema=w.ema, scale=w.scale,
                               score_mode=mode))
        inputs.append(inp)
        apps.append(wl.make_append_tokens(w, "cuda"))
    return layers, inputs, apps


def _snapshot(layer):
    return {"scores": layer.scores.clone(), "A": layer.A.lists(), "M": layer.M.lists(),
            "acc": layer.state.acc.clone(), "l": layer.state.l.clone(), "m": layer.state.m.clone(),
            "out": layer.out.clone()}


def _predictor(layer):
    return {"level": layer.level.clone(), "trend": layer.trend.clone(), "live": layer.live.clone(),
            "P": layer.P_cur.lists()}


def _equal(a, b, what):
    for k in a:
        if isinstance(a[k], torch.Tensor):
            assert torch.equal(a[k], b[k]), f"{what}: {k}"
        else:
            assert a[k] == b[k], f"{what}: {k}"


@pytest.mark.parametrize("which", ["all", "one_layer"])
def test_stack_equals_layers_run_alone(which):
    steps = 5
    specs = _workloads(steps)
    if which == "one_layer":
        specs = specs[:1]
    stack_layers, s_inp, s_app = _build(specs)
    ref_layers, r_inp, r_app = _build(specs)
    stack = PRRStack(stack_layers)
    L = len(specs)
    for t in range(steps):
        qs = [s_inp[i].q[t] for i in range(L)]
        stack.step(qs, [s_app[i][0][t] for i in range(L)], [s_app[i][1][t] for i in range(L)])
        for i, layer in enumerate(ref_layers):
            layer.append(r_app[i][0][t], r_app[i][1][t])
            layer.step(r_inp[i].q[t])
        torch.cuda.synchronize()
        for i in range(L):
            _equal(_snapshot(stack_layers[i]), _snapshot(ref_layers[i]), f"step {t} layer {i}")
            assert torch.equal(s_inp[i].seq_len, r_inp[i].seq_len)
            # every layer's predictor except the pending one has run by now
            if i != stack.pending_owner:
                _equal(_predictor(stack_layers[i]), _predictor(ref_layers[i]), f"step {t} layer {i} predictor")
    stack.flush()
    torch.cuda.synchronize()
    for i in range(L):
        _equal(_predictor(stack_layers[i]), _predictor(ref_layers[i]), f"final predictor layer {i}")
    # the trajectory exercised the carried predictor: the sets differ from step to step
    assert any(len(p) for row in stack_layers[0].P_cur.lists() for p in row)


def test_carried_predictor_equals_predict_alone():
    """prr_select_spec_predict = prr_select_spec followed by prr_predict, for a carried row inside the
    launch and one after it."""
    specs = _workloads(2)
    for carrier, carried in ((0, 2), (2, 1)):
        layers, inp, _ = _build([specs[carrier], specs[carried]])
        Y, X = layers
        X.step(inp[1].q[0], defer_predict=True)
        args = X.take_pending_predict()
        torch.cuda.synchronize()
        lv, tr, live = args.level.clone(), args.trend.clone(), args.live.clone()
        B, H = X.live.shape
        Pref = bd.BlockSet.empty(B, H, args.budget, lv.device)
        bd.predict(args.scores, args.seq_len, args.block, args.alpha, args.beta, args.gamma, args.budget, lv,
                   tr, live, P_next=Pref)
        ref = bd.select_spec(inp[0].q[0], Y.kv, Y.meta, Y.block, Y.topk, Y.P_cur, Y.scale, mode=Y.score_mode)
        got = bd.select_spec(inp[0].q[0], Y.kv, Y.meta, Y.block, Y.topk, Y.P_cur, Y.scale, mode=Y.score_mode,
                             pred=args)
        torch.cuda.synchronize()
        assert torch.equal(ref[0], got[0])
        assert ref[1].lists() == got[1].lists() and ref[2].lists() == got[2].lists()
        for x, y in ((ref[3].acc, got[3].acc), (ref[3].l, got[3].l), (ref[3].m, got[3].m)):
            assert torch.equal(x, y)
        assert torch.equal(args.level, lv) and torch.equal(args.trend, tr) and torch.equal(args.live, live)
        assert args.P_next.lists() == Pref.lists()
        # the first pair carries a row inside the launch, the second one too long for it
        assert (X.nmax <= 2048) == (carried == 2)
