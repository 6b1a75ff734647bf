"""prr_spec_attn_noalloc (the speculative pass on the library's own per-GPU buffer, for callers that cannot
allocate) against prr_spec_attn with a workspace of the caller's: two calls in a row, the second on a
smaller input and another stream, both bit for bit equal to the workspace entry point (same kernel, same
chunking); a set too large for the buffer is refused before anything is enqueued."""
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


def _random_sets(w, cap, n, seed):
    rng = np.random.default_rng(seed)
    nb = w.blocks_of(0)
    return [[sorted(rng.choice(nb, size=min(n, nb), replace=False).tolist()) for _ in range(w.num_kv_heads)]
            for _ in range(w.batch)]


def _compare(w, cap, n, seed, stream=None):
    print(f"[noalloc] B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} T={w.context} "
          f"S={w.block} cap={cap} |P|={n}", flush=True)
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    P = sets_to_device(_random_sets(w, cap, n, seed), cap)
    ref = bd.spec_attn(inp.q[0], kv, w.block, P, w.scale)
    got = bd.AttnState.empty(w.batch, w.num_q_heads, w.head_dim)
    if stream is None:
        bd.spec_attn_noalloc(inp.q[0], kv, w.block, P, w.scale, out=got)
    else:
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            bd.spec_attn_noalloc(inp.q[0], kv, w.block, P, w.scale, out=got, stream=stream)
        torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for name in ("acc", "l", "m"):
        assert torch.equal(getattr(ref, name), getattr(got, name)), name


def test_two_calls_in_a_row_second_smaller():
    big = wl.Workload("noalloc_big", 4, 32, 8, 128, 65536, 64, 64, "bf16", seed=51)
    small = wl.Workload("noalloc_small", 1, 8, 2, 64, 8192, 32, 16, "bf16", seed=52)
    _compare(big, 64, 64, seed=1)
    _compare(small, 16, 11, seed=2, stream=torch.cuda.Stream())


def test_set_too_large_for_the_buffer_is_refused():
    w = wl.Workload("noalloc_refused", 4, 32, 8, 128, 4096, 64, 8, "bf16", seed=53)
    inp = wl.make_inputs(w, "cuda")
    kv = device_kv(inp)
    cap = 4096   # 2048 chunks per unit: far beyond the buffer
    need = bd.attn_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block, cap)
    assert need > 16 << 20
    P = bd.BlockSet.empty(w.batch, w.num_kv_heads, cap, "cuda")
    with pytest.raises(bd.PrrError) as e:
        bd.spec_attn_noalloc(inp.q[0], kv, w.block, P, w.scale)
    assert e.value.status == 3   # PRR_EWORKSPACE
