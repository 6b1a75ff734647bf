"""One PRR decode layer step on three HIP streams (orchestration only; all compute is in libprr.so).

The speculative pass over the predicted set P runs on a side stream while Quest selection runs on the
critical stream; repair waits for both.  The predictor needs only the selection's scores, so it runs on a
third stream next to repair, off the critical path ([paper] §1 and Figure 1 flow, §3: speculation
overlaps selection, repair handles M = A \\ P after it; [paper] §4.1 predictor and A.5: prediction is off
the critical path).

Citations: [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context
LLM Decoding" (full paper text).

Stream order per step (no host synchronisation, no device-to-host copy):
  critical:  wait(e_pred: P^t written) -> record e_ready -> select(q^t, P^t) -> A^t, M^t, IS^t
             -> record e_sel;  wait(e_spec) -> repair(M^t) -> O^t
  side:      wait(e_ready) -> spec_attn(P^t) -> record e_spec   (submitted after select)
  predictor: wait(e_sel) -> predict(IS^t) -> P^{t+1} (the other P buffer) -> record e_pred
At the first step P is empty, so repair computes plain block-sparse attention over A.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import binding as bd


@dataclass
class StepTimers:
    """Optional timing events, recorded on the stream each kernel runs on."""

    start: torch.cuda.Event
    select_end: torch.cuda.Event
    spec_start: torch.cuda.Event
    spec_end: torch.cuda.Event
    repair_start: torch.cuda.Event
    repair_end: torch.cuda.Event
    predict_start: torch.cuda.Event
    predict_end: torch.cuda.Event

    @staticmethod
    def make() -> "StepTimers":
        return StepTimers(*[torch.cuda.Event(enable_timing=True) for _ in range(8)])


class PRRLayer:
    """Device state of one attention layer for a batch: paged cache, block metadata, predictor state,
    block sets (P double-buffered), attention state and workspaces."""

    def __init__(self, kv: bd.KVCache, num_q_heads: int, block: int, topk: int, budget: int,
                 ema=(0.6, 0.3, 0.5), scale: Optional[float] = None,
                 side_stream: Optional[torch.cuda.Stream] = None,
                 predict_stream: Optional[torch.cuda.Stream] = None):
        dev = kv.k.device
        self.kv = kv
        self.hq = num_q_heads
        self.block = block
        self.topk = topk
        self.budget = budget
        self.alpha, self.beta, self.gamma = (float(x) for x in ema)
        self.scale = float(scale) if scale is not None else kv.head_dim ** -0.5
        B, H, d = kv.batch, kv.num_kv_heads, kv.head_dim
        self.meta = bd.build_meta(kv, block)
        self.nmax = bd.max_blocks(kv, block)
        self.scores = torch.zeros((B, H, self.nmax), dtype=torch.float64, device=dev)
        self.level = torch.zeros_like(self.scores)
        self.trend = torch.zeros_like(self.scores)
        self.live = torch.zeros((B, H), dtype=torch.int32, device=dev)
        self.P = [bd.BlockSet.empty(B, H, max(1, budget), dev), bd.BlockSet.empty(B, H, max(1, budget), dev)]
        self.cur = 0
        self.A = bd.BlockSet.empty(B, H, max(1, topk), dev)
        self.M = bd.BlockSet.empty(B, H, max(1, topk), dev)
        self.state = bd.AttnState.empty(B, num_q_heads, d, dev)
        self.out = torch.zeros((B, num_q_heads, d), dtype=torch.float32, device=dev)
        self.ws_spec = bd.workspace_for(kv, num_q_heads, block, max(1, budget))
        self.ws_repair = bd.workspace_for(kv, num_q_heads, block, max(1, topk))
        self.side = side_stream if side_stream is not None else torch.cuda.Stream(device=dev)
        self.aux = predict_stream if predict_stream is not None else torch.cuda.Stream(device=dev)
        self.e_ready = torch.cuda.Event()
        self.e_spec = torch.cuda.Event()
        self.e_sel = torch.cuda.Event()
        self.e_pred = torch.cuda.Event()
        self.e_pred.record(self.aux)

    @property
    def P_cur(self) -> bd.BlockSet:
        return self.P[self.cur]

    def reset(self):
        """Forget the predictor state (a fresh decode: the first step runs with P empty)."""
        torch.cuda.current_stream().wait_event(self.e_pred)
        self.level.zero_()
        self.trend.zero_()
        self.live.zero_()
        for p in self.P:
            p.count.zero_()
        self.cur = 0

    def step(self, q: torch.Tensor, timers: Optional[StepTimers] = None) -> torch.Tensor:
        """Enqueue one layer step for queries q [B][Hq][d]; returns the normalised output tensor
        (valid once the critical stream reaches it)."""
        crit = torch.cuda.current_stream()
        side, aux = self.side, self.aux
        P = self.P[self.cur]
        Pn = self.P[1 - self.cur]
        if timers:
            timers.start.record(crit)
        crit.wait_event(self.e_pred)          # P^t written by the previous step's predictor
        self.e_ready.record(crit)             # q, P^t and the previous repair's state are in place
        side.wait_event(self.e_ready)
        # selection is submitted first so that its workgroups are dispatched ahead of the speculative
        # pass, which would otherwise fill every SIMD and push selection behind it
        bd.select(q, self.kv, self.meta, self.block, self.topk, P=P, scores=self.scores, A=self.A,
                  M=self.M, stream=crit)
        self.e_sel.record(crit)
        if timers:
            timers.select_end.record(crit)
            timers.spec_start.record(side)
        bd.spec_attn(q, self.kv, self.block, P, self.scale, out=self.state, ws=self.ws_spec, stream=side)
        if timers:
            timers.spec_end.record(side)
        self.e_spec.record(side)
        aux.wait_event(self.e_sel)
        if timers:
            timers.predict_start.record(aux)
        bd.predict(self.scores, self.kv.seq_len, self.block, self.alpha, self.beta, self.gamma, self.budget,
                   self.level, self.trend, self.live, P_next=Pn, stream=aux)
        if timers:
            timers.predict_end.record(aux)
        self.e_pred.record(aux)
        crit.wait_event(self.e_spec)
        if timers:
            timers.repair_start.record(crit)
        bd.repair(q, self.kv, self.block, self.M, self.scale, self.state, out=self.out, ws=self.ws_repair,
                  stream=crit)
        if timers:
            timers.repair_end.record(crit)
        self.cur = 1 - self.cur
        return self.out
