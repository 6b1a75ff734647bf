"""bench.py's oracle timing on the CPU: the one-thread leg and the worker-process leg run the same
speculative attention and repair work on a small workload and report consistent figures."""
import os
import sys

from block_sparse_attention_quest_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import bench
    return bench


def test_cpu_baseline_one_thread_and_worker_processes():
    bench = _bench()
    w = wl.scaled(wl.C3, context=4096, batch=1)
    inp = wl.make_inputs(w, "cpu")
    units, steps = 3, 3
    pool = bench.OraclePool(2)
    try:
        r = bench.cpu_baseline(inp, w, units, steps, pool=pool)
    finally:
        pool.close()
    assert all(not p.is_alive() for p in pool.procs)
    assert r["kind"] == "oracle" and r["cores"] == 2
    assert r["value"] > 0 and r["value_one_thread"] > 0 and r["seconds_attn"] > 0
    # both legs time the same bytes: their ratio is the ratio of their times
    ratio = r["value"] / r["value_one_thread"]
    assert abs(ratio - r["seconds_attn_one_thread"] / r["seconds_attn"]) <= 0.02 * ratio + 1e-3


def test_cpu_baseline_without_pool_is_the_one_thread_leg():
    bench = _bench()
    w = wl.scaled(wl.C3, context=4096, batch=1)
    inp = wl.make_inputs(w, "cpu")
    r = bench.cpu_baseline(inp, w, 2, 2)
    assert r["cores"] == 1 and r["value"] == r["value_one_thread"]


def test_budget_profile_rejects_lengths_that_clip_the_largest_budget():
    """A profiled length must hold max(delta) K blocks, else that point measures a clipped budget; the
    check runs before any GPU work."""
    import argparse

    import pytest

    bench = _bench()
    w = wl.C3   # K = 64 blocks of 64 tokens
    args = argparse.Namespace(budget_profile="8192,65536", budget_deltas="0.5,1,4", budget_check="",
                              budget_degree=1, budget_reps=1)
    with pytest.raises(ValueError, match=r"\[8192\]"):   # 128 blocks < 4 x 64
        bench.budget_profile(args, w, None, None)
    args.budget_profile, args.budget_check = "16384,65536", "12288"
    with pytest.raises(ValueError, match=r"\[12288\]"):
        bench.budget_profile(args, w, None, None)


def test_oracle_pool_calibration_deals_the_grid_and_matches_the_oracle():
    """The calibration leg's all-core oracle run: candidates dealt round-robin to the workers come back in
    grid order and equal the oracle's own grid search."""
    import numpy as np

    from oracle import prr_oracle as orc

    bench = _bench()
    IS = wl.make_calibration_scores(wl.C5, rows=40, blocks=48).astype(np.float64)
    grid = orc.calibration_grid()
    pool = bench.OraclePool(3)
    try:
        wall, H = pool.calibrate(IS, 8, grid)
    finally:
        pool.close()
    ref, _ = orc.calibrate(IS, 8, grid)
    assert wall > 0 and np.array_equal(H, ref)
