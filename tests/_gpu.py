"""Helpers shared by the GPU parity tests: device inputs, per-unit oracle views, state comparison."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

# Tolerances on floating-point state (bf16 KV, fp32 accumulation): O max abs 5e-3, l relative 1e-4,
# m relative 1e-4 (absolute below |m| = 1).
O_TOL = 5e-3
L_TOL = 1e-4
M_TOL = 1e-4


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def device_kv(inp: wl.Inputs) -> bd.KVCache:
    return bd.KVCache(inp.k_cache, inp.v_cache, inp.page_table, inp.seq_len)


def sets_to_device(sets, cap, device="cuda") -> bd.BlockSet:
    """Nested lists [b][kvh] -> BlockSet with the given capacity."""
    B, H = len(sets), len(sets[0])
    idx = np.zeros((B, H, cap), dtype=np.int32)
    cnt = np.zeros((B, H), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            s = np.asarray(sets[b][h], dtype=np.int32)
            idx[b, h, :s.size] = s
            cnt[b, h] = s.size
    return bd.BlockSet(torch.from_numpy(idx).to(device), torch.from_numpy(cnt).to(device))


def unit_view(inp: wl.Inputs, b: int, kvh: int, step: int = 0, length: int = None):
    """Oracle inputs of one (sequence, kv head) unit: q [1][G][d] float64 and a one-sequence,
    one-kv-head PagedKV with an identity page table (layout only)."""
    w = inp.w
    length = w.lengths[b] if length is None else length
    G = w.group
    pages = inp.page_table[b].long()
    k = wl.to_numpy_bits(inp.k_cache[pages, kvh].unsqueeze(1))
    v = wl.to_numpy_bits(inp.v_cache[pages, kvh].unsqueeze(1))
    n = pages.numel()
    kv = orc.make_paged_kv(k, v, np.arange(n).reshape(1, n), np.array([length]), w.dtype)
    q = orc.upcast(wl.to_numpy_bits(inp.q[step, b, kvh * G:(kvh + 1) * G]), w.dtype)[None]
    return q, kv


def unit_meta(kv: orc.PagedKV, block: int):
    return orc.build_meta(kv, block, 1)[0][0]


def assert_state(acc, l, m, ref: orc.State, what=""):
    """GPU state (acc [d], l, m as numpy / floats) against an oracle state."""
    acc = np.asarray(acc, dtype=np.float64)
    l = float(l)
    m = float(m)
    if ref.l == 0.0:
        assert l == 0.0 and m == -math.inf and np.all(acc == 0.0), what
        return
    assert abs(l - ref.l) <= L_TOL * ref.l, f"{what}: l {l} vs {ref.l}"
    assert abs(m - ref.m) <= M_TOL * max(1.0, abs(ref.m)), f"{what}: m {m} vs {ref.m}"
    err = np.max(np.abs(acc / l - ref.out))
    assert err <= O_TOL, f"{what}: max |O - O_ref| = {err}"


def assert_heads(state: bd.AttnState, refs: dict, what=""):
    """refs: {(b, h): State}"""
    acc = state.acc.double().cpu().numpy()
    l = state.l.double().cpu().numpy()
    m = state.m.double().cpu().numpy()
    for (b, h), ref in refs.items():
        assert_state(acc[b, h], l[b, h], m[b, h], ref, f"{what} b={b} h={h}")
