#!/usr/bin/env python3
"""Benchmark of the PRR decode hot path on one MI355X.

Workload (default): 128K context, batch 8, 32 query / 8 kv heads, head_dim 128, block 64, K = 64
blocks, bf16, a drifting query trajectory (AR(1), rho 0.9, ~68% adjacent top-K overlap) with the EMA
predictor (alpha 0.6, beta 0.3, gamma 0.5) producing P.  Decode step 0 runs with P empty (untimed);
each timed step t >= 1 does, on synthetic inputs already resident in HBM:

  1. flush (a 1 GiB read: evicts L2 and the 256 MB MALL, as a decode step's other layers would),
     then the layer step on one stream: select_spec (scoring || spec_attn(P^t) in one grid, then top-K)
     -> repair(M^t) -> predict, with an event after each;
  2. flush, an empty event pair (the cost of the two event records themselves);
     flush, spec_attn(P^t) alone;  flush, repair(M^t) alone;  flush, select alone;  flush, predict alone
     (on copies of the predictor state);  flush, select_spec alone.
The trajectory is then replayed twice: the single-stream step (the reported us per layer step: the start
of the selection + speculative kernel to the end of the repair kernel) and, for comparison, the pages'
three-stream schedule (select on the critical stream, spec_attn on a side stream, predict on a third).

Kernel time = the GPU time of a call's kernels, read from HIP events bound to the launches themselves
(prr_time_next_kernel: hipExtLaunchKernel with start/stop events; the start of the call's first kernel
to the end of its last), so no event-record cost is in it; the same figures rocprofv3's kernel trace
reports.  Event pairs recorded around each call are reported beside them (*_raw).  value = effective KV
GB/s of spec-attn + repair = algorithmic KV bytes ((|P| + |M|) * block * head_dim * 2 tensors * 2 B,
summed over (sequence, kv head) units) / (spec kernel time + repair kernel time).

Also reported: us per layer step, per-kernel us, |M|, overlap and hit rate, the roofline
of the dominant kernel (spec-attn), and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E peak
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "spec_attn_ctx128k_b8_hbm_counters.md")
PROFILE_KERNEL_STATS = os.path.join(ROOT, "profiles", "attn_ctx128k_b8_kernel_stats.md")
PROFILE_WORKLOAD = "ctx128k_b8_64steps"   # the workload (fixed context) those profiles were taken on


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=63)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="ctx128k_b8_64steps")
    ap.add_argument("--flush-mib", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the calibration leg of workloads that have a prefill score matrix (their steps then "
                         "use the workload's default EMA parameters)")
    ap.add_argument("--cpu-units", type=int, default=64, help="(sequence, kv head) units in the CPU sample")
    ap.add_argument("--cpu-steps", type=int, default=0, help="decode steps in the CPU sample (0: all timed)")
    ap.add_argument("--stack", type=int, default=0,
                    help="also time a stack of this many layers (own caches and predictor state each) with each "
                         "layer's predictor carried by the next layer's launch, against the same layers run "
                         "with the predictor on its own")
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8"), default=None,
                    help="cache element type (default: the workload's, bf16); fp8 = E4M3 K/V with bf16 queries")
    ap.add_argument("--layer-step", choices=("one", "two"), default="one",
                    help="the layer step as one launch (prr_layer_step) or as prr_select_spec + prr_repair")
    ap.add_argument("--score-mode", choices=("quest", "mean"), default="quest",
                    help="block summary selection scores: Quest's min/max bound or the block's mean key")
    ap.add_argument("--append", action="store_true",
                    help="decode-loop mode: every timed step first appends one token per sequence (prr_append, "
                         "timed alone) so the context grows by one token per step")
    ap.add_argument("--delta-sweep", default="",
                    help="comma-separated speculation budgets |P| = delta K to time as extra layer steps "
                         "(e.g. 1,1.25,1.5,2); empty: none")
    ap.add_argument("--delta-steps", type=int, default=24, help="decode steps timed per delta")
    ap.add_argument("--budget-profile", default="",
                    help="comma-separated context lengths (tokens): profile selection and speculative-attention "
                         "latency over them and --budget-deltas, fit the budget table and report its choices "
                         "(e.g. 16384,32768,65536,131072; every length must hold the largest budget, max(delta) K blocks); "
                         "empty: none")
    ap.add_argument("--budget-deltas", default="0.25,0.5,0.75,1,1.5,2,3,4",
                    help="budget ratios |P| = delta K profiled by --budget-profile")
    ap.add_argument("--budget-degree", type=int, default=1,
                    help="degree of the budget table's regression (selection reads metadata in proportion to the "
                         "context and speculation is flat in it, so lines extrapolate best)")
    ap.add_argument("--budget-check", default="98304,262144,524288",
                    help="off-grid context lengths where the table's estimates are compared with measurements")
    ap.add_argument("--budget-reps", type=int, default=20, help="timed runs per profiled point")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size (HBM counter calibration under rocprofv3)")
    return ap.parse_args()


def kv_bytes_per_block(w) -> int:
    return w.block * w.kv_bytes_per_token()


def algorithmic_bytes(w, score_mode: str, spec_bytes, rep_bytes) -> dict:
    """Algorithmic HBM bytes per launch of each kernel of the path (medians over the timed steps where
    they depend on the sets), for the HBM-counter summaries' traffic ratios:
      spec / repair: the K/V of the set's blocks (block x 2 x d x element bytes per block);
      score: the metadata scoring reads, d elements per block (the one row, min or max, that the sign of
             qbar_i picks per channel; the fp32 mean for mean-pooled scoring), plus the 8-byte score written;
      topk: the 8-byte scores read; predict: scores, level and trend read and level and trend written
             (8 bytes each);
      select_spec = score + spec; layer_step = score + spec + repair.
    Sets, lengths and queries (a few KiB) are left out."""
    import numpy as np

    blocks = sum(w.blocks_of(b) for b in range(w.batch)) * w.num_kv_heads
    elem = 4 if (score_mode == "mean" or w.dtype == "f32") else 2
    score = blocks * (w.head_dim * elem + 8)
    spec, rep = float(np.median(spec_bytes)), float(np.median(rep_bytes))
    return {"spec": spec, "repair": rep, "score": float(score), "topk": float(blocks * 8),
            "predict": float(blocks * 40), "select_spec": score + spec, "layer_step": score + spec + rep}


def load_profile_value(path: str, kernel_hash: str, key: str):
    """A "- key: value" line of a committed profile summary, or None when the file is absent, lacks the
    key or was taken on a different attention kernel source."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_hash:
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def load_traffic(kernel_hash: str):
    """HBM bytes per spec-attn launch from the committed counter summary, or None when absent or
    taken on a different kernel source."""
    return load_profile_value(PROFILE_COUNTERS, kernel_hash, "hbm_bytes_per_launch")


def _cpu_unit_view(inp, w, b, h):
    """Oracle view of one (sequence, kv head) unit: its pages only, upcast to float64."""
    import numpy as np

    from block_sparse_attention_quest_amd import workloads as wl
    from oracle import prr_oracle as orc

    pages = inp.page_table[b].long()
    k = wl.to_numpy_bits(inp.k_cache[pages, h].unsqueeze(1))
    v = wl.to_numpy_bits(inp.v_cache[pages, h].unsqueeze(1))
    n = pages.numel()
    return orc.make_paged_kv(k, v, np.arange(n).reshape(1, n), np.array([w.lengths[b]]), w.dtype)


def _oracle_worker(conn):
    """A CPU worker of the oracle timing: keeps the units it is sent (cache bits upcast to an oracle
    view, queries, recorded sets) and, on "run", times speculative attention over P and repair over M
    for every recorded step of every unit it holds.  BLAS runs on one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import prr_oracle as orc

    held = []
    with threadpool_limits(limits=1):
        while True:
            cmd, payload = conn.recv()
            try:
                if cmd == "load":
                    k, v, length, dtype, block, scale, G, qs, sets = payload
                    n = k.shape[0]
                    kv = orc.make_paged_kv(k, v, np.arange(n).reshape(1, n), np.array([length]), dtype)
                    held.append((kv, block, scale, G, qs, sets))
                    conn.send(("ok", None))
                elif cmd == "calib":
                    IS, k, grid = payload
                    t0 = time.perf_counter()
                    H, _ = orc.calibrate(IS, k, grid)
                    conn.send(("ok", (time.perf_counter() - t0, H)))
                elif cmd == "run":
                    t0 = time.perf_counter()
                    for kv, block, scale, G, qs, sets in held:
                        for t, (P, M) in enumerate(sets):
                            q = qs[t][None]
                            for g in range(G):
                                orc.merge(orc.head_state(q, kv, 0, g, G, P, block, scale),
                                          orc.head_state(q, kv, 0, g, G, M, block, scale))
                    conn.send(("ok", time.perf_counter() - t0))
                else:
                    conn.send(("ok", None))
                    return
            except Exception as e:  # reported to the parent, which stops the timing
                conn.send(("error", repr(e)))


class OraclePool:
    """Worker processes for the oracle timing, forked before anything touches the GPU (the children
    never use it); each holds the oracle views of the units it is sent."""

    def __init__(self, n: int):
        import multiprocessing as mp

        ctx = mp.get_context("fork")
        self.conns, self.procs = [], []
        for _ in range(n):
            a, b = ctx.Pipe()
            proc = ctx.Process(target=_oracle_worker, args=(b,), daemon=True)
            proc.start()
            self.conns.append(a)
            self.procs.append(proc)

    def _reply(self, i, timeout=900.0):
        c = self.conns[i]
        if not c.poll(timeout):
            raise RuntimeError(f"oracle worker {i} did not answer within {timeout} s")
        status, val = c.recv()
        if status != "ok":
            raise RuntimeError(f"oracle worker {i}: {val}")
        return val

    def load(self, i, payload):
        self.conns[i].send(("load", payload))
        self._reply(i)

    def run(self) -> float:
        """Wall time of one timed pass of every worker over the units it holds."""
        t0 = time.perf_counter()
        for c in self.conns:
            c.send(("run", None))
        for i in range(len(self.conns)):
            self._reply(i)
        return time.perf_counter() - t0

    def calibrate(self, IS, k, grid):
        """The oracle's grid search with the candidates dealt round-robin to the workers (each ranks the
        rows' true top-K sets itself, as the oracle does); returns (wall seconds, H in grid order)."""
        import numpy as np

        W = len(self.conns)
        shares = [list(range(i, len(grid), W)) for i in range(W)]
        t0 = time.perf_counter()
        for i, c in enumerate(self.conns):
            if shares[i]:
                c.send(("calib", (IS, k, grid[shares[i]])))
        H = np.zeros(len(grid))
        for i in range(W):
            if shares[i]:
                _, h = self._reply(i)
                H[shares[i]] = h
        return time.perf_counter() - t0, H

    def close(self):
        for i, c in enumerate(self.conns):
            try:
                c.send(("exit", None))
                self._reply(i, timeout=30.0)
            except Exception:
                pass
        for proc in self.procs:
            proc.join(timeout=10)
            if proc.is_alive():
                proc.terminate()


def cpu_baseline(inp, w, units, steps, score_mode="quest", pool=None):
    """Time the oracle on a bounded sample of the same workload: `units` (sequence, kv head) pairs for
    decode steps 0..steps (step 0 has P empty and is not counted), BLAS limited to one thread.  Block
    metadata is built once per unit before timing, as on the GPU.
      1. One thread runs every stage (selection, speculative attention, repair, predictor) unit by unit
         and records each step's sets P and M.
      2. The same attention work (spec over P, repair over M) on all host cores: `pool`'s worker
         processes (one per core, forked before the GPU was touched) each hold a share of the units'
         oracle views, built before the timed region; the wall time of one pass of all of them.
    value is the effective-KV-GB/s of the second leg on `cores` processes (of the first, on one core,
    without a pool); the one-thread figures are kept beside it."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from block_sparse_attention_quest_amd import workloads as wl
    from oracle import prr_oracle as orc

    G = w.group
    alpha, beta, gamma = w.ema
    t_attn = t_all = 0.0
    nbytes = 0
    n_unit_steps = 0
    pairs = [(u // w.num_kv_heads, u % w.num_kv_heads) for u in range(units)]
    recorded = {}
    qsteps = {}
    with threadpool_limits(limits=1):
        for b, h in pairs:
            kv = _cpu_unit_view(inp, w, b, h)
            if score_mode == "quest":
                mn, mx = orc.build_meta(kv, w.block, 1)[0][0]
            else:
                mean = orc.build_mean_meta(kv, w.block, 1)[0][0]
            lv, tr, live, P = np.zeros(0), np.zeros(0), 0, np.zeros(0, dtype=np.int64)
            qs = orc.upcast(wl.to_numpy_bits(inp.q[: steps + 1, b, h * G:(h + 1) * G]), w.dtype)
            qsteps[(b, h)] = qs[1:]
            recorded[(b, h)] = []
            for t in range(steps + 1):
                q = qs[t][None]
                t0 = time.perf_counter()
                qbar = orc.representative_query(q, 0, 0, G)
                s = orc.quest_scores(qbar, mn, mx) if score_mode == "quest" else orc.mean_scores(qbar, mean)
                A = orc.topk_blocks(s, w.topk)
                M = orc.set_minus(A, P)
                t1 = time.perf_counter()
                states = [orc.head_state(q, kv, 0, g, G, list(P), w.block, w.scale) for g in range(G)]
                states = [orc.merge(st, orc.head_state(q, kv, 0, g, G, list(M), w.block, w.scale))
                          for g, st in enumerate(states)]
                t2 = time.perf_counter()
                nbytes += (len(P) + len(M)) * kv_bytes_per_block(w) if t >= 1 else 0
                if t >= 1:
                    recorded[(b, h)].append((list(P), list(M)))
                lv, tr, live, P = orc.predict_step(lv, tr, live, s, alpha, beta, gamma, w.topk)
                t3 = time.perf_counter()
                if t >= 1:
                    t_attn += t2 - t1
                    t_all += t3 - t0
                    n_unit_steps += 1
            del kv
        W, wall = 1, t_attn
        if pool is not None:
            W = len(pool.conns)
            for i, (b, h) in enumerate(pairs):
                pages = inp.page_table[b].long()
                k = wl.to_numpy_bits(inp.k_cache[pages, h].unsqueeze(1))
                v = wl.to_numpy_bits(inp.v_cache[pages, h].unsqueeze(1))
                pool.load(i % W, (k, v, w.lengths[b], w.dtype, w.block, w.scale, G, qsteps[(b, h)],
                                  recorded[(b, h)]))
            wall = pool.run()
    return {
        "value": round(nbytes / wall / 1e9, 4) if wall > 0 else None,
        "unit": "effective KV GB/s (spec-attn + repair)",
        "cores": W,
        "kind": "oracle",
        "sample": f"{units} (sequence, kv head) units x {steps} decode steps of the same workload "
                  f"(float64 NumPy); value: spec + repair of every unit-step on {W} processes (units dealt "
                  f"round-robin, BLAS one thread each); value_one_thread: the same work on one thread",
        "seconds_attn": round(wall, 3),
        "value_one_thread": round(nbytes / t_attn / 1e9, 4) if t_attn > 0 else None,
        "seconds_attn_one_thread": round(t_attn, 3),
        "seconds_all_stages_one_thread": round(t_all, 3),
        "us_per_unit_step_attn_one_thread": round(t_attn / max(1, n_unit_steps) * 1e6, 1),
        "us_per_unit_step_all_one_thread": round(t_all / max(1, n_unit_steps) * 1e6, 1),
        "cpu_count_visible": len(os.sched_getaffinity(0)),
    }


class EventPool:
    """Timing events made before a timed region.  torch creates a HIP event at its first record, and a
    creation can hold the host for milliseconds; when the GPU has drained its queue meanwhile, the stall
    lands between two timing events.  reserve(n) creates n events (one record each) up front; calling
    the pool hands them out."""

    def __init__(self):
        self.free = []

    def reserve(self, n: int):
        import torch

        s = torch.cuda.current_stream()
        for _ in range(max(0, n - len(self.free))):
            e = torch.cuda.Event(enable_timing=True)
            e.record(s)
            self.free.append(e)
        torch.cuda.synchronize()

    def __call__(self):
        import torch

        return self.free.pop() if self.free else torch.cuda.Event(enable_timing=True)


def calibration_leg(w, flush, ev, pool, oracle: bool = True, reps: int = 10, sample: int = 4):
    """Online predictor calibration of the workload's prefill score matrix ([paper] §4.2; [blog] Eqs. (4)-(5)):
    prr_calibrate timed on the GPU (the span of its kernels, after the flush; median of `reps`), and the
    oracle's grid search timed beside it: on one core over `sample` of the candidates (the rows' true top-K
    sets, which every candidate shares, timed apart and counted once in the full-grid estimate), and over the
    whole grid on the worker processes.  Returns (report, theta*)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from block_sparse_attention_quest_amd import binding as bd
    from block_sparse_attention_quest_amd import workloads as wl
    from oracle import prr_oracle as orc

    IS = wl.make_calibration_scores(w)
    rows, blocks = IS.shape
    s = torch.from_numpy(IS).cuda()
    grid = bd.calibration_grid("cuda")
    n = grid.shape[0]
    ws = bd.Workspace(bd.load_library().prr_calibrate_workspace_bytes(rows, blocks, n))
    H, best = bd.calibrate(s, w.topk, grid, ws=ws)   # first launches load the code objects
    torch.cuda.synchronize()
    ev.reserve(2 * reps)
    pairs = []
    for _ in range(reps):
        flush()
        k0, k1 = ev(), ev()
        bd.time_next_kernel(k0, k1)
        H, best = bd.calibrate(s, w.topk, grid, ws=ws)
        pairs.append((k0, k1))
    torch.cuda.synchronize()
    gpu_us = [a.elapsed_time(b) * 1e3 for a, b in pairs]
    Hh = H.cpu().numpy()
    j = int(best.cpu().numpy()[0])
    theta = tuple(float(x) for x in grid[j].cpu().numpy())
    rep = {"rows": rows, "blocks": blocks, "k": w.topk, "candidates": n, "theta_star": list(theta),
           "best_index": j, "H_star": round(float(Hh[j]), 9),
           "gpu_us_median": round(float(statistics.median(gpu_us)), 2),
           "gpu_us_p10_p90": [round(float(np.percentile(gpu_us, 10)), 2), round(float(np.percentile(gpu_us, 90)), 2)]}
    if not oracle:
        return rep, theta
    IS64 = IS.astype(np.float64)
    ogrid = orc.calibration_grid()
    picks = np.linspace(0, n - 1, sample).round().astype(int)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for phi in range(rows):
            orc.topk_blocks(IS64[phi], w.topk)
        t_sets = time.perf_counter() - t0
        t0 = time.perf_counter()
        oH, _ = orc.calibrate(IS64, w.topk, ogrid[picks])
        t_sample = time.perf_counter() - t0
    per_cand = max(t_sample - t_sets, 0.0) / sample
    rep["oracle_one_core"] = {"seconds_sample": round(t_sample, 3), "sample_candidates": [int(x) for x in picks],
                              "seconds_true_sets": round(t_sets, 3),
                              "seconds_full_grid_estimate": round(t_sets + n * per_cand, 2),
                              "H_sample_matches_gpu": bool(np.all(np.abs(oH - Hh[picks]) <= 1e-9 * oH))}
    if pool is not None:
        wall, Hall = pool.calibrate(IS64, w.topk, ogrid)
        rep["oracle_all_cores"] = {"cores": len(pool.conns), "seconds_full_grid": round(wall, 2),
                                   "best_index": int(np.argmax(Hall)),
                                   "H_matches_gpu": bool(np.all(np.abs(Hall - Hh) <= 1e-9 * Hall))}
    rep["note"] = ("gpu: prr_calibrate, first kernel start to last kernel end; oracle: float64 NumPy, one "
                   "process per core; the pages quote 2.4 ms (16K prefill) and 11.2 ms (64K) for the same "
                   "80-point search on an unnamed CPU, overlapped with prefill (context only)")
    return rep, theta


def delta_sweep(args, w, inp, kv, meta, flush, ev):
    """Layer-step time against the speculation budget |P| = delta K (the pages' critical-path-aware budget):
    for each delta, a fresh trajectory (step 0 untimed), then `delta_steps` lean one-stream steps."""
    import numpy as np
    import torch

    from block_sparse_attention_quest_amd.layer_step import PRRLayer, StepTimers

    out = []
    n = min(args.delta_steps, w.steps - 1)
    for d in [float(x) for x in args.delta_sweep.split(",") if x.strip()]:
        budget = max(1, int(round(d * w.topk)))
        L = PRRLayer(kv, w.num_q_heads, w.block, w.topk, budget, ema=w.ema, scale=w.scale,
                     fused=args.layer_step == "one")
        for t in range(3):
            L.step(inp.q[t])
        torch.cuda.synchronize()
        L.reset()
        L.step(inp.q[0])
        ev.reserve(2 * n)
        times, hits, missed, pc = [], [], [], []
        for i in range(n):
            P = L.P_cur
            flush()
            tm = StepTimers(None, None, None, None, ev(), ev())
            L.step(inp.q[1 + i], tm)
            torch.cuda.synchronize()
            times.append(tm.kernel_start.elapsed_time(tm.kernel_end) * 1e3)
            a = L.A.idx.cpu().numpy()
            p_idx, p_cnt = P.idx.cpu().numpy(), P.count.cpu().numpy()
            mc = L.M.count.cpu().numpy()
            for b in range(w.batch):
                for h in range(w.num_kv_heads):
                    hits.append(len(set(a[b, h].tolist()) & set(p_idx[b, h, :p_cnt[b, h]].tolist())) / w.topk)
            missed.append(float(mc.mean()))
            pc.append(float(p_cnt.mean()))
        out.append({"delta": d, "budget_blocks": budget, "us_layer_step_median": round(float(np.median(times)), 2),
                    "hit_rate": round(float(np.mean(hits)), 4), "mean_missed_blocks": round(float(np.mean(missed)), 2),
                    "mean_P_blocks": round(float(np.mean(pc)), 2), "steps": n})
        del L
        log(f"[bench] delta {d}: {out[-1]}")
    return out


def _budget_point(w, T, deltas, reps, flush, ev, seed):
    """Median selection latency and speculative-attention latency at each delta for the workload's shape
    at T tokens (each run after the cache flush; the GPU time of the call's kernels, prr_time_next_kernel).  P at delta is a
    seeded random set of round(delta K) distinct blocks per (sequence, kv head)."""
    import numpy as np
    import torch

    from block_sparse_attention_quest_amd import binding as bd
    from block_sparse_attention_quest_amd import workloads as wl

    wt = wl.scaled(w, context=T, steps=2, append_tokens=0)
    inp = wl.make_inputs(wt, "cuda")
    kv = bd.KVCache(inp.k_cache, inp.v_cache, inp.page_table, inp.seq_len)
    meta = bd.build_meta(kv, wt.block)
    B, H, N = wt.batch, wt.num_kv_heads, bd.max_blocks(kv, wt.block)
    budgets = [max(1, min(N, int(round(d * wt.topk)))) for d in deltas]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    order = torch.argsort(torch.rand((B, H, N), generator=gen, device="cuda"), dim=-1).to(torch.int32)
    sets = []
    for nb in budgets:
        idx = torch.sort(order[..., :nb], dim=-1).values.contiguous()
        sets.append(bd.BlockSet(idx, torch.full((B, H), nb, dtype=torch.int32, device="cuda")))
    ws = bd.workspace_for(kv, wt.num_q_heads, wt.block, max(budgets))
    state = bd.AttnState.empty(B, wt.num_q_heads, wt.head_dim, "cuda")
    scores = torch.zeros((B, H, N), dtype=torch.float64, device="cuda")
    A = bd.BlockSet.empty(B, H, wt.topk, "cuda")
    M = bd.BlockSet.empty(B, H, wt.topk, "cuda")
    q = inp.q[0]
    P1 = sets[min(range(len(deltas)), key=lambda j: abs(deltas[j] - 1.0))]
    crit = torch.cuda.current_stream()

    def timed(fn):
        ev.reserve(2 * reps)
        pairs = []
        for _ in range(reps):
            flush()
            k0, k1 = ev(), ev()
            bd.time_next_kernel(k0, k1)
            fn()
            pairs.append((k0, k1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) * 1e3 for a, b in pairs]))

    for P in sets:   # warm every shape once
        bd.spec_attn(q, kv, wt.block, P, wt.scale, out=state, ws=ws)
    ws_sel = bd.select_workspace_for(kv, wt.block, wt.topk)
    bd.select(q, kv, meta, wt.block, wt.topk, P=P1, scores=scores, A=A, M=M, ws=ws_sel)
    t_sel = timed(lambda: bd.select(q, kv, meta, wt.block, wt.topk, P=P1, scores=scores, A=A, M=M, stream=crit,
                                    ws=ws_sel))
    t_spec = [timed(lambda P=P: bd.spec_attn(q, kv, wt.block, P, wt.scale, out=state, ws=ws, stream=crit))
              for P in sets]
    del inp, kv, meta, order, sets, ws, state, scores
    torch.cuda.empty_cache()
    return t_sel, t_spec, budgets


def budget_profile(args, w, flush, ev):
    """The pages' critical-path-aware budget (§4.4, A.6): profile selection and speculative-attention
    latency over context lengths and budget ratios, fit the library's budget table, and report the
    largest delta whose speculative pass ends no later than selection at each profiled length and at
    off-grid lengths (where the estimates are also compared with measurements)."""
    from block_sparse_attention_quest_amd import binding as bd

    ctx = [int(x) for x in args.budget_profile.split(",") if x.strip()]
    deltas = [float(x) for x in args.budget_deltas.split(",") if x.strip()]
    check = [int(x) for x in args.budget_check.split(",") if x.strip()]
    short = [T for T in ctx + check if -(-T // w.block) < int(round(max(deltas) * w.topk))]
    if short:
        # a budget larger than the context is clipped to every block: that point measures no delta
        raise ValueError(f"context lengths {short} hold fewer than max(delta) K = "
                         f"{int(round(max(deltas) * w.topk))} blocks of {w.block} tokens")
    sel, spec = [], [[] for _ in deltas]
    for i, T in enumerate(ctx):
        t_sel, t_spec, budgets = _budget_point(w, T, deltas, args.budget_reps, flush, ev, seed=100 + i)
        sel.append(t_sel)
        for j, t in enumerate(t_spec):
            spec[j].append(t)
        log(f"[bench] budget profile T={T}: select {t_sel:.2f} us, spec {[round(t, 2) for t in t_spec]} us")
    tab = bd.BudgetTable([float(T) for T in ctx], sel, deltas, spec, args.budget_degree)

    def pick(T):
        j, est = tab.choose(float(T))
        return {"context": T, "delta": deltas[j] if j >= 0 else None, "choice": j,
                "est_us_select": round(float(est[0]), 2),
                "est_us_spec": [round(float(e), 2) for e in est[1:]]}

    choices = [pick(T) for T in ctx]
    checks = []
    for i, T in enumerate(check):
        c = pick(T)
        t_sel, t_spec, _ = _budget_point(w, T, deltas, args.budget_reps, flush, ev, seed=200 + i)
        c["measured_us_select"] = round(t_sel, 2)
        c["measured_us_spec"] = [round(t, 2) for t in t_spec]
        fits = [j for j, t in enumerate(t_spec) if t <= t_sel]
        c["measured_choice"] = max(fits) if fits else -1
        checks.append(c)
        log(f"[bench] budget check T={T}: {c}")
    return {"ctx": ctx, "deltas": deltas, "budget_blocks_at_K": [max(1, int(round(d * w.topk))) for d in deltas],
            "us_select": [round(t, 2) for t in sel], "us_spec": [[round(t, 2) for t in r] for r in spec],
            "degree": args.budget_degree, "coef": tab.coef.tolist(), "choices": choices, "checks": checks,
            "note": "kernels timed alone, after the cache flush (first kernel start to last kernel end); selection = "
                    "prr_select (scores, top-K, M), speculation = prr_spec_attn over round(delta K) blocks"}


def measure_stack(args, w, layer0, inp0, flush, ev):
    """Decode steps through args.stack layers of the workload's shape (layer 0 is the main layer, the others
    get inputs of their own seeds): per-layer time with the predictor carried by the next layer's launch
    (PRRStack) against the same layers with the predictor as its own launch.  The cache is flushed before
    every layer, outside the timed region."""
    import torch

    from block_sparse_attention_quest_amd import binding as bd
    from block_sparse_attention_quest_amd import workloads as wl
    from block_sparse_attention_quest_amd.layer_step import PRRLayer, PRRStack, StepTimers

    L, K = args.stack, args.steps
    layers, qs = [layer0], [inp0.q]
    for i in range(1, L):
        wi = wl.scaled(w, seed=w.seed + 1000 * i)
        inp = wl.make_inputs(wi, layer0.kv.k.device)
        kv = bd.KVCache(inp.k_cache, inp.v_cache, inp.page_table, inp.seq_len)
        layers.append(PRRLayer(kv, w.num_q_heads, w.block, w.topk, w.topk, ema=w.ema, scale=w.scale,
                               score_mode=args.score_mode, fused=args.layer_step == "one"))
        qs.append(inp.q)
        del inp
    torch.cuda.synchronize()
    log(f"[bench] stack of {L} layers ready")
    el = lambda a, b: a.elapsed_time(b) * 1e3

    def run(carried: bool, K: int):
        ev.reserve(2 * L * K)
        for layer in layers:
            layer.reset()
        stack = PRRStack(layers)
        for layer in layers:   # decode step 0 (P empty), not timed
            layer.step(qs[layers.index(layer)][0])
        torch.cuda.synchronize()
        per_layer = []
        for i in range(K):
            t = 1 + i
            if carried:
                tms = [StepTimers(ev(), None, ev(), None) for _ in range(L)]
                stack.step([q[t] for q in qs], timers=tms, before_layer=lambda l: flush())
                per_layer.append([(tm.start, tm.repair_end) for tm in tms])
            else:
                row = []
                for li, layer in enumerate(layers):
                    flush()
                    tm = StepTimers(ev(), None, None, ev())
                    layer.step(qs[li][t], tm)
                    row.append((tm.start, tm.predict_end))
                per_layer.append(row)
        stack.flush()
        torch.cuda.synchronize()
        return [el(a, b) for row in per_layer for a, b in row]

    run(True, 2)   # first launches of the carrying kernels (code object loads), not timed
    alone = run(False, K)
    carried = run(True, K)
    for layer in layers[1:]:
        del layer
    med = lambda xs: round(float(statistics.median(xs)), 2)
    return {"layers": L, "us_per_layer_carried_median": med(carried), "us_per_layer_alone_median": med(alone),
            "note": "per layer: carried = start of its select_spec (which also runs the previous layer's "
                    "predictor) to the end of its repair; alone = start of select_spec to the end of its own "
                    "predictor launch; both one stream, cache flushed before every layer"}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the PRR hot path here is built and "
              "measured on a single GPU, and multi-GPU runs are out of scope.", file=sys.stderr)
        sys.exit(2)

    # the oracle timing's worker processes are forked before anything touches the GPU
    pool = OraclePool(min(16, len(os.sched_getaffinity(0)))) if not args.no_cpu_baseline else None

    import numpy as np
    import torch

    from block_sparse_attention_quest_amd import binding as bd
    from block_sparse_attention_quest_amd import profiling
    from block_sparse_attention_quest_amd import workloads as wl
    from block_sparse_attention_quest_amd.layer_step import PRRLayer, StepTimers, TwoStreamTimers

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    bd.load_library()
    dev = torch.device("cuda:0")
    K = args.steps
    base = wl.CONFIGS[args.config]
    w = wl.scaled(base, steps=max(base.steps, args.warmup + 1, K + 1),
                  append_tokens=(K + 1) if args.append else 0, dtype=args.kv_dtype or base.dtype)
    log(f"[bench] generating {w.name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"T={w.context} S={w.block} K={w.topk} steps={w.steps}")
    t_gen = time.time()
    inp = wl.make_inputs(w, dev)
    kv = bd.KVCache(inp.k_cache, inp.v_cache, inp.page_table, inp.seq_len)
    layer = PRRLayer(kv, w.num_q_heads, w.block, w.topk, w.topk, ema=w.ema, scale=w.scale,
                     score_mode=args.score_mode, fused=args.layer_step == "one")
    if args.append:
        k_app, v_app = wl.make_append_tokens(w, dev)
        len0 = inp.seq_len.clone()
    torch.cuda.synchronize()
    log(f"[bench] inputs + metadata ready in {time.time() - t_gen:.1f}s")

    flush_buf = torch.empty(args.flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    flush_buf.fill_(1.0)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_sink)

    ev = EventPool()
    calib = None
    if w.calib_rows and not args.no_calibration:
        # the workload's predictor parameters come from calibration over its prefill score matrix
        log(f"[bench] calibrating on the {w.calib_rows} x {w.calib_blocks} prefill score matrix")
        calib, theta = calibration_leg(w, flush, ev, pool, oracle=not args.no_cpu_baseline)
        w = wl.scaled(w, ema=theta)
        layer.alpha, layer.beta, layer.gamma = theta
        log(f"[bench] theta* = {theta}; calibration {calib['gpu_us_median']} us on the GPU")

    # isolated-measurement buffers (the layer's own sets and state stay untouched)
    B, H = w.batch, w.num_kv_heads
    iso_state = bd.AttnState.empty(B, w.num_q_heads, w.head_dim, dev)
    iso_scores = torch.zeros_like(layer.scores)
    iso_A = bd.BlockSet.empty(B, H, w.topk, dev)
    iso_M = bd.BlockSet.empty(B, H, w.topk, dev)
    ws_iso_spec = bd.select_spec_workspace_for(kv, w.num_q_heads, w.block, w.topk, w.topk)
    ws_iso_rep = bd.workspace_for(kv, w.num_q_heads, w.block, w.topk)
    iso_level, iso_trend = torch.empty_like(layer.level), torch.empty_like(layer.trend)
    iso_live = torch.empty_like(layer.live)
    iso_P = bd.BlockSet.empty(B, H, w.topk, dev)
    ws_iso_pred = bd.predict_workspace_for(B, H, layer.nmax, w.topk, dev)

    # warmup: a few layer steps and every call the timed loop isolates (a kernel's first launch in the
    # process loads its code object, milliseconds that would land in one timed step), then start the
    # trajectory afresh
    for t in range(args.warmup):
        q = inp.q[t % w.steps]
        layer.step(q)
        P = layer.P_cur
        bd.spec_attn(q, kv, w.block, P, w.scale, out=iso_state, ws=ws_iso_spec)
        bd.repair(q, kv, w.block, layer.M, w.scale, iso_state, ws=ws_iso_rep)
        bd.select(q, kv, layer.meta, w.block, w.topk, P=P, scores=iso_scores, A=iso_A, M=iso_M,
                  mode=args.score_mode, ws=layer.ws_select)
        bd.select_spec(q, kv, layer.meta, w.block, w.topk, P, w.scale, scores=iso_scores, A=iso_A, M=iso_M,
                       out=iso_state, ws=ws_iso_spec, mode=args.score_mode)
        iso_level.copy_(layer.level)
        iso_trend.copy_(layer.trend)
        iso_live.copy_(layer.live)
        bd.predict(layer.scores, kv.seq_len, w.block, *w.ema, w.topk, iso_level, iso_trend, iso_live, P_next=iso_P,
                   ws=ws_iso_pred)
        flush()
    torch.cuda.synchronize()
    layer.reset()
    layer.step(inp.q[0])          # decode step 0: P empty (plain DSA through repair), not timed
    torch.cuda.synchronize()
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    crit = torch.cuda.current_stream()
    iso_names = ("empty", "spec", "repair", "select", "predict", "select_spec")
    ev.reserve(K * (6 + 4 * len(iso_names)))
    rec = []
    p_counts = torch.zeros((K, B, H), dtype=torch.int32, device=dev)
    m_counts = torch.zeros_like(p_counts)
    a_sets = torch.zeros((K, B, H, w.topk), dtype=torch.int32, device=dev)
    p_sets = torch.zeros_like(a_sets)
    append_pairs = []

    torch.cuda.synchronize()
    gc.disable()   # no collector pauses between a kernel and its timing event
    wall0 = time.perf_counter()
    for i in range(K):
        t = 1 + i
        q = inp.q[t]
        P = layer.P_cur
        if args.append:
            flush()
            e0, e1, k0, k1 = ev(), ev(), ev(), ev()
            e0.record(crit)
            bd.time_next_kernel(k0, k1)
            layer.append(k_app[i], v_app[i], stream=crit)
            e1.record(crit)
            append_pairs.append((e0, e1, k0, k1))
        # 1. layer step with a breakdown (events after each call) and its kernel span
        flush()
        tm = StepTimers(ev(), ev(), ev(), ev(), ev(), ev())
        layer.step(q, tm)
        p_counts[i].copy_(P.count)
        m_counts[i].copy_(layer.M.count)
        a_sets[i].copy_(layer.A.idx)
        p_sets[i].copy_(P.idx)
        # 2. isolated, each after a flush, on the same sets: an empty event pair, then each call with an
        #    event pair around it (dispatch and completion included) and events bound to its kernels
        #    (prr_time_next_kernel: the start of its first kernel, the end of its last)
        pairs = []
        iso_level.copy_(layer.level)
        iso_trend.copy_(layer.trend)
        iso_live.copy_(layer.live)
        for what in iso_names:
            flush()
            e0, e1, k0, k1 = ev(), ev(), ev(), ev()
            e0.record(crit)
            if what != "empty":
                bd.time_next_kernel(k0, k1)
            if what == "spec":
                bd.spec_attn(q, kv, w.block, P, w.scale, out=iso_state, ws=ws_iso_spec, stream=crit)
            elif what == "repair":
                bd.repair(q, kv, w.block, layer.M, w.scale, iso_state, ws=ws_iso_rep, stream=crit)
            elif what == "select":
                bd.select(q, kv, layer.meta, w.block, w.topk, P=P, scores=iso_scores, A=iso_A, M=iso_M,
                          mode=args.score_mode, stream=crit, ws=layer.ws_select)
            elif what == "predict":
                bd.predict(layer.scores, kv.seq_len, w.block, *w.ema, w.topk, iso_level, iso_trend, iso_live,
                           P_next=iso_P, ws=ws_iso_pred, stream=crit)
            elif what == "select_spec":
                bd.select_spec(q, kv, layer.meta, w.block, w.topk, P, w.scale, scores=iso_scores, A=iso_A,
                               M=iso_M, out=iso_state, ws=ws_iso_spec, mode=args.score_mode, stream=crit)
            e1.record(crit)
            pairs.append((e0, e1, k0, k1))
        rec.append((tm, *pairs))
        if (i + 1) % 16 == 0:
            log(f"[bench] {i + 1}/{K} steps enqueued")
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    def replay(two_streams: bool):
        """Replay the trajectory with a start and an end event per step only (and, on one stream, the
        kernel span: the start of the selection + speculative kernel to the end of repair)."""
        layer.reset()
        if args.append:   # back to the initial context: lengths, then the metadata of every block
            inp.seq_len.copy_(len0)
            (bd.build_meta if args.score_mode == "quest" else bd.build_mean_meta)(kv, w.block, layer.meta)
        layer.step(inp.q[0])
        ev.reserve(4 * K)
        out = []
        for i in range(K):
            if args.append:
                layer.append(k_app[i], v_app[i], stream=crit)
            flush()
            if two_streams:
                tm = TwoStreamTimers(ev(), None, None, None, None, ev())
                layer.step_two_streams(inp.q[1 + i], tm)
                out.append((tm.start, tm.repair_end, None, None))
            else:
                tm = StepTimers(ev(), None, ev(), None, ev(), ev())
                layer.step(inp.q[1 + i], tm)
                out.append((tm.start, tm.repair_end, tm.kernel_start, tm.kernel_end))
        torch.cuda.synchronize()
        return out

    lean_one = replay(False)
    lean_two = replay(True)

    def el(a, b):
        return a.elapsed_time(b) * 1e3   # microseconds

    # per call: raw = the event pair around it; kernel = the span of its kernels (prr_time_next_kernel)
    iso_raw = {nm: [el(r[1 + j][0], r[1 + j][1]) for r in rec] for j, nm in enumerate(iso_names)}
    iso_us = {nm: [el(r[1 + j][2], r[1 + j][3]) for r in rec] for j, nm in enumerate(iso_names) if nm != "empty"}
    base_us = float(statistics.median(iso_raw["empty"]))
    spec_raw, rep_raw = iso_raw["spec"], iso_raw["repair"]
    spec_us, rep_us = iso_us["spec"], iso_us["repair"]
    step_lean_us = [el(a, b) for a, b, _, _ in lean_one]
    step_kernel_us = [el(c, d) for _, _, c, d in lean_one]
    step_two_us = [el(a, b) for a, b, _, _ in lean_two]
    step_tm_us = [el(r[0].start, r[0].repair_end) for r in rec]
    ss_ov_us = [el(r[0].start, r[0].select_spec_end) for r in rec]
    rep_ov_us = [el(r[0].select_spec_end, r[0].repair_end) for r in rec]
    pred_ov_us = [el(r[0].repair_end, r[0].predict_end) for r in rec]

    pc = p_counts.cpu().numpy().astype(np.int64)
    mc = m_counts.cpu().numpy().astype(np.int64)
    per_blk = kv_bytes_per_block(w)
    spec_bytes = pc.reshape(K, -1).sum(1) * per_blk
    rep_bytes = mc.reshape(K, -1).sum(1) * per_blk
    tot_bytes = float(spec_bytes.sum() + rep_bytes.sum())
    value = tot_bytes / ((sum(spec_us) + sum(rep_us)) * 1e-6) / 1e9
    value_raw = tot_bytes / ((sum(spec_raw) + sum(rep_raw)) * 1e-6) / 1e9
    spec_gbps = float(spec_bytes.sum() / (sum(spec_us) * 1e-6) / 1e9)
    rep_gbps = float(rep_bytes.sum() / (sum(rep_us) * 1e-6) / 1e9)
    step_gbps = [(sb + rb) / ((a + b) * 1e-6) / 1e9 for sb, rb, a, b in zip(spec_bytes, rep_bytes, spec_us, rep_us)]
    algo_bytes = algorithmic_bytes(w, args.score_mode, spec_bytes, rep_bytes)

    A_all = a_sets.cpu().numpy()
    P_all = p_sets.cpu().numpy()
    overlaps, hits = [], []
    for i in range(K):
        for b in range(B):
            for h in range(H):
                a = set(A_all[i, b, h].tolist())
                if i:
                    overlaps.append(len(a & set(A_all[i - 1, b, h].tolist())) / w.topk)
                hits.append(len(a & set(P_all[i, b, h, :pc[i, b, h]].tolist())) / w.topk)

    kernel_hash = profiling.kernel_source_hash()
    spec_launch_bytes = float(spec_bytes.mean())
    spec_launch_us = float(statistics.mean(spec_us))
    achieved = spec_launch_bytes / (spec_launch_us * 1e-6) / 1e9
    # the committed counters were taken on the default run (Quest scoring, no appends)
    traffic = (load_traffic(kernel_hash)
               if (w.name == PROFILE_WORKLOAD and not args.append and args.score_mode == "quest"
                   and w.dtype == "bf16") else None)

    rocprof_ref = {"rocprof_avg_launch_us": None, "rocprof_frac": None}
    if w.name == PROFILE_WORKLOAD and not args.append and args.score_mode == "quest" and w.dtype == "bf16":
        avg = load_profile_value(PROFILE_KERNEL_STATS, kernel_hash, "attn_spec_avg_us")
        if avg:
            rocprof_ref = {"rocprof_avg_launch_us": avg,
                           "rocprof_frac": round(spec_launch_bytes / (avg * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    med = lambda xs: round(float(statistics.median(xs)), 2)
    result = {
        "metric": "effective KV GB/s (frac of HBM peak) + us/layer-step, spec-attn+repair",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "context": w.context, "block": w.block, "topk_blocks": w.topk,
                   "spec_budget_blocks": w.topk, "ema": list(w.ema), "decode_steps_timed": K,
                   "score_mode": args.score_mode, "kv_dtype": w.dtype,
                   "layer_step": "one launch" if args.layer_step == "one" else "select_spec + repair",
                   "parallelism": "none (1 GPU)", "flush_mib_read_between_kernels": args.flush_mib},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "value_median_step_gbps": round(float(statistics.median(step_gbps)), 1),
        "value_note": "value = all timed steps' KV bytes / their summed spec + repair kernel time (one slow step "
                      "counts in full); value_median_step_gbps = the median step's own figure",
        "timing_note": "kernel us = the GPU time of a call's kernels, from HIP events bound to them "
                       "(prr_time_next_kernel: hipExtLaunchKernel with start/stop events, the start of the first "
                       "kernel to the end of the last), each call alone after the same flush; *_raw figures are "
                       "event pairs recorded around the call (they add the event records' own cost)",
        "us_empty_event_pair_median": round(base_us, 2),
        "value_raw_events_gbps": round(value_raw, 1),
        "us_per_layer_step_median": med(step_kernel_us),
        "us_per_layer_step_p10_p90": [round(float(np.percentile(step_kernel_us, 10)), 2),
                                      round(float(np.percentile(step_kernel_us, 90)), 2)],
        "layer_step_note": "one stream: the start of the selection + speculative kernel to the end of the repair "
                           "kernel (events bound to the kernels); the predictor follows repair on the same stream "
                           "(off this path)",
        "us_per_layer_step_events_median": med(step_lean_us),
        "us_per_layer_step_two_streams_median": med(step_two_us),
        "us_spec_attn_median": med(spec_us),
        "us_spec_attn_p10_p90": [round(float(np.percentile(spec_us, 10)), 2),
                                 round(float(np.percentile(spec_us, 90)), 2)],
        "us_spec_attn_max": round(float(max(spec_us)), 2),
        "us_repair_max": round(float(max(rep_us)), 2),
        "us_repair_median": med(rep_us),
        "us_repair_p10_p90": [round(float(np.percentile(rep_us, 10)), 2),
                              round(float(np.percentile(rep_us, 90)), 2)],
        "us_select_median": med(iso_us["select"]),
        "us_select_spec_median": med(iso_us["select_spec"]),
        "us_select_plus_spec_median": med([a + b for a, b in zip(iso_us["select"], spec_us)]),
        "us_predict_median": med(iso_us["predict"]),
        "raw_event_us_median": {nm: med(xs) for nm, xs in iso_raw.items()},
        "in_layer_step": {"us_select_spec_median": med(ss_ov_us), "us_repair_median": med(rep_ov_us),
                          "us_predict_median": med(pred_ov_us), "us_to_repair_end_median": med(step_tm_us),
                          "note": "one stream with an event after each call (the events add their own cost)"},
        "algorithmic_bytes_per_launch": {k: round(v) for k, v in algo_bytes.items()},
        "spec_attn_gbps": round(spec_gbps, 1),
        "repair_gbps": round(rep_gbps, 1),
        "mean_missed_blocks_per_unit": round(float(mc.mean()), 2),
        "adjacent_overlap": round(float(np.mean(overlaps)), 4),
        "hit_rate": round(float(np.mean(hits)), 4),
        "ms_per_step_note": "wall time per timed step of the first pass: one layer step + isolated empty pair, "
                            "spec, repair, select, predict and select_spec, each after a 1 GiB cache flush",
        "roofline": {"bound": "hbm", "kernel": f"attn_spec_{w.dtype}<{w.head_dim}>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": spec_launch_bytes,
                     "avg_launch_us": round(spec_launch_us, 2), "kernel_source_sha256": kernel_hash,
                     "avg_launch_note": "mean over the timed steps of the kernel's own duration (HIP events bound "
                                        "to the launch); rocprof_* = the committed rocprofv3 kernel trace of the "
                                        "same kernel source (null when the source differs)",
                     **rocprof_ref},
    }
    if args.append:
        result["decode_append"] = {
            "us_append_median": round(float(statistics.median([el(k0, k1) for _, _, k0, k1 in append_pairs])), 2),
            "note": "each timed step appends one token per sequence before its layer step (context grows "
                    "by one token per step); append time = the append kernel's own duration"}
        if args.delta_sweep:
            log("[bench] --delta-sweep is skipped in --append mode")
            args.delta_sweep = ""
    if calib is not None:
        result["calibration"] = calib
    if args.delta_sweep:
        result["delta_sweep"] = delta_sweep(args, w, inp, kv, layer.meta, flush, ev)
    if args.budget_profile:
        result["budget"] = budget_profile(args, w, flush, ev)
    if args.stack > 1 and not args.append:
        result["stack"] = measure_stack(args, w, layer, inp, flush, ev)
    if not args.no_cpu_baseline:
        steps = args.cpu_steps if args.cpu_steps > 0 else K
        units = min(args.cpu_units, B * H)
        log(f"[bench] timing the CPU oracle on {units} units x {steps} steps")
        try:
            result["cpu_baseline"] = cpu_baseline(inp, w, units, steps, args.score_mode, pool)
        finally:
            pool.close()
    gc.enable()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
