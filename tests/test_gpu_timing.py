"""Kernel timing through the C ABI (prr_time_next_kernel): events bound to a call's kernels.

The timing only changes how the kernels are launched (hipExtLaunchKernel with the armed events), so the
results must be bit-for-bit those of an untimed call; the kernel span must be positive and shorter than
an event pair recorded around the same call; a call consumes the arming (the next call is untimed); and
a call that launches several kernels is timed from the first kernel's start to the last kernel's end.
"""
import pytest
import torch

from _gpu import device_kv, require_gpu
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


def _ev():
    e = torch.cuda.Event(enable_timing=True)
    e.record()
    return e


def _setup():
    w = wl.Workload("timing", 2, 16, 4, 128, 16384, 32, 32, "bf16", seed=91)
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    meta = bd.build_meta(kv, w.block)
    _, A, _ = bd.select(inp.q[0], kv, meta, w.block, w.topk)
    return w, inp, kv, meta, A


def test_timed_spec_attn_is_bitwise_the_untimed_one():
    w, inp, kv, meta, A = _setup()
    plain = bd.spec_attn(inp.q[0], kv, w.block, A, w.scale)
    k0, k1, e0, e1 = _ev(), _ev(), _ev(), _ev()
    torch.cuda.synchronize()
    e0.record()
    bd.time_next_kernel(k0, k1)
    timed = bd.spec_attn(inp.q[0], kv, w.block, A, w.scale)
    e1.record()
    torch.cuda.synchronize()
    for name in ("acc", "l", "m"):
        assert torch.equal(getattr(plain, name), getattr(timed, name)), name
    kern = k0.elapsed_time(k1) * 1e3
    outer = e0.elapsed_time(e1) * 1e3
    print(f"[timing] spec_attn kernel {kern:.2f} us, event pair {outer:.2f} us", flush=True)
    assert 0.0 < kern <= outer


def test_arming_is_consumed_by_one_call():
    w, inp, kv, meta, A = _setup()
    k0, k1 = _ev(), _ev()
    torch.cuda.synchronize()
    bd.time_next_kernel(k0, k1)
    bd.spec_attn(inp.q[0], kv, w.block, A, w.scale)
    torch.cuda.synchronize()
    first = k0.elapsed_time(k1)
    # the next calls are not timed: the events keep the first call's times
    bd.spec_attn(inp.q[0], kv, w.block, A, w.scale)
    bd.repair(inp.q[0], kv, w.block, A, w.scale, bd.AttnState.empty(w.batch, w.num_q_heads, w.head_dim))
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == first


def test_multi_kernel_call_spans_first_to_last_kernel():
    """prr_select launches the scoring kernel and then the top-K kernel; a timed call gives the same sets
    and a positive span (the start of the first kernel to the end of the last)."""
    w, inp, kv, meta, A = _setup()
    k0, k1, s0, s1 = _ev(), _ev(), _ev(), _ev()
    torch.cuda.synchronize()
    base = s0.elapsed_time(s1)
    bd.time_next_kernel(k0, k1)
    scores, A2, _ = bd.select(inp.q[0], kv, meta, w.block, w.topk)
    torch.cuda.synchronize()
    assert A2.lists() == A.lists()
    assert k0.elapsed_time(k1) > 0.0
    # a call that fails its argument checks consumes the arming and records nothing: the next call is
    # untimed and the events keep their earlier records
    bd.time_next_kernel(s0, s1)
    with pytest.raises(bd.PrrError):
        bd.select(inp.q[0], kv, meta, w.block, -1)
    bd.select(inp.q[0], kv, meta, w.block, w.topk)
    torch.cuda.synchronize()
    assert s0.elapsed_time(s1) == base
