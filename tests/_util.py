"""Test helpers: turn generated inputs into oracle inputs, and compare results."""
import numpy as np

from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc


def oracle_view(inp: "wl.Inputs"):
    """(q [steps][B][Hq][d] float64, PagedKV) from generated torch inputs."""
    w = inp.w
    q = orc.upcast(wl.to_numpy_bits(inp.q), w.dtype)
    kv = orc.make_paged_kv(wl.to_numpy_bits(inp.k_cache), wl.to_numpy_bits(inp.v_cache),
                           wl.to_numpy_bits(inp.page_table), wl.to_numpy_bits(inp.seq_len), w.dtype)
    return q, kv


def random_disjoint_sets(rng, n_blocks, n_a, n_b):
    """Two disjoint random block sets of sizes n_a and n_b (as python lists)."""
    perm = rng.permutation(n_blocks)
    return list(perm[:n_a]), list(perm[n_a:n_a + n_b])


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.maximum(np.abs(b), 1e-300)
    return float(np.max(np.abs(a - b) / den)) if a.size else 0.0
