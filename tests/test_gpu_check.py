"""Checking mode (PRR_CHECK=1): set entries out of range, repeated entries and counts beyond the
capacity are reported as PRR_EINVAL before any attention or selection work is enqueued; valid sets run
as usual.  The mode is read once per process, so the checks run in a child process of their own."""
import os
import subprocess
import sys

import pytest

from _gpu import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys
import torch
sys.path.insert(0, "tests")
from _gpu import device_kv, sets_to_device
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl

w = wl.Workload("check", 2, 8, 2, 128, 1000, 16, 8, "bf16", seed=5, seq_lens=[1000, 600])   # 63 and 38 blocks
inp = wl.make_inputs(w, "cuda")
kv = device_kv(inp)
meta = bd.build_meta(kv, w.block)
good = [[[1, 5, 9], [0, 62]], [[37], []]]
cases = {
    "repeat": [[[1, 5, 1], [0, 62]], [[37], []]],
    "range": [[[1, 5, 9], [0, 62]], [[38], []]],      # sequence 1 has 38 blocks: 0 .. 37
    "negative": [[[1, -1], [0]], [[3], []]],
}

def expect_einval(fn, what):
    try:
        fn()
    except bd.PrrError as e:
        assert e.status == 1, (what, e.status)
        return
    raise AssertionError(f"{what}: accepted")

for name, sets in cases.items():
    S = sets_to_device(sets, 8)
    st = bd.spec_attn(inp.q[0], kv, w.block, sets_to_device(good, 8), w.scale)
    expect_einval(lambda: bd.spec_attn(inp.q[0], kv, w.block, S, w.scale), "spec " + name)
    expect_einval(lambda: bd.repair(inp.q[0], kv, w.block, S, w.scale, st), "repair " + name)
    expect_einval(lambda: bd.select(inp.q[0], kv, meta, w.block, w.topk, P=S), "select " + name)
    expect_einval(lambda: bd.select_spec(inp.q[0], kv, meta, w.block, w.topk, S, w.scale), "select_spec " + name)
over = sets_to_device(good, 8)
over.count[0, 0] = 9                                   # count beyond the capacity
expect_einval(lambda: bd.spec_attn(inp.q[0], kv, w.block, over, w.scale), "count")
# valid sets run, and give what they give without the checks
G = sets_to_device(good, 8)
a = bd.spec_attn(inp.q[0], kv, w.block, G, w.scale)
scores, A, M, b = bd.select_spec(inp.q[0], kv, meta, w.block, w.topk, G, w.scale)
torch.cuda.synchronize()
assert torch.equal(a.acc, b.acc) and torch.equal(a.l, b.l) and torch.equal(a.m, b.m)
print("CHECKS OK", flush=True)
'''


def test_checking_mode_rejects_bad_sets():
    require_gpu()
    env = dict(os.environ, PRR_CHECK="1")
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0 and "CHECKS OK" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
