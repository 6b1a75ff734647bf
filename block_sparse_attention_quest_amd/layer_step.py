"""One PRR decode layer step (orchestration only; all compute is in libprr.so).

The method runs the speculative pass over the predicted set P concurrently with Quest selection, then
repairs the state with the missed blocks M = A \\ P; the predictor needs only the selection's scores and
is off the critical path ([paper] §1 and the Figure 1 flow, §3; [paper] §4.1 and A.5).

Citations: [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context
LLM Decoding" (full paper text).

Two schedules of the same work, with identical results:

* ``step`` (the default): one stream.  ``prr_layer_step`` runs scoring, the speculative pass and repair in
  one grid (their workgroups share the GPU, so the overlap happens inside the launch, and the repair of a
  (sequence, kv head) starts as soon as its top-K is known), then the predictor:
      layer_step(q^t, P^t) -> A^t, M^t, IS^t, O^t  ->  predict(IS^t) -> P^{t+1}
  With fused=False at construction: ``prr_select_spec`` (scoring and the speculative pass in one grid, the
  top-K), then ``prr_repair``, then the predictor.  On this GPU a dependency between two streams costs
  about 10 us from the producer's end to the consumer's start, against about 1 us between kernels of one
  stream, so the one-stream schedules are the fast ones.
* ``step_two_streams``: the pages' schedule on three streams (selection on the critical stream, the
  speculative pass on a side stream, the predictor on a third), joined by events.  Kept to measure the
  difference.

Neither synchronises with the host or copies to it.  At the first step P is empty, so repair computes
plain block-sparse attention over A.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import binding as bd


@dataclass
class StepTimers:
    """Optional timing events of ``step`` (all on the one stream); a field left None is not recorded.
    kernel_start / kernel_end are bound to kernels (prr_time_next_kernel): the start of the selection +
    speculative kernel and the end of the repair kernel, so their span is the step's GPU time without the
    cost of event records."""

    start: Optional[torch.cuda.Event]
    select_spec_end: Optional[torch.cuda.Event]
    repair_end: Optional[torch.cuda.Event]
    predict_end: Optional[torch.cuda.Event]
    kernel_start: Optional[torch.cuda.Event] = None
    kernel_end: Optional[torch.cuda.Event] = None

    @staticmethod
    def make() -> "StepTimers":
        return StepTimers(*[torch.cuda.Event(enable_timing=True) for _ in range(6)])

    @staticmethod
    def lean() -> "StepTimers":
        """Start and end of repair only (no event between the calls)."""
        return StepTimers(torch.cuda.Event(enable_timing=True), None, torch.cuda.Event(enable_timing=True), None)


@dataclass
class TwoStreamTimers:
    """Optional timing events of ``step_two_streams``, each on the stream its kernel runs on; a field left
    None is not recorded."""

    start: Optional[torch.cuda.Event]
    select_end: Optional[torch.cuda.Event]
    spec_start: Optional[torch.cuda.Event]
    spec_end: Optional[torch.cuda.Event]
    repair_start: Optional[torch.cuda.Event]
    repair_end: Optional[torch.cuda.Event]

    @staticmethod
    def make() -> "TwoStreamTimers":
        return TwoStreamTimers(*[torch.cuda.Event(enable_timing=True) for _ in range(6)])


class PRRLayer:
    """Device state of one attention layer for a batch: paged cache, block metadata, predictor state,
    block sets (P double-buffered), attention state and workspaces.

    score_mode "quest" scores blocks by Quest's bound over channel-wise min/max keys; "mean" by the
    product of the representative query with each block's mean key (the two block summaries the pages
    name for selection).  The metadata kept in ``meta`` is the one the mode reads."""

    def __init__(self, kv: bd.KVCache, num_q_heads: int, block: int, topk: int, budget: int,
                 ema=(0.6, 0.3, 0.5), scale: Optional[float] = None, score_mode: str = "quest",
                 max_budget: Optional[int] = None, fused: bool = True, page_lists: bool = True):
        dev = kv.k.device
        # |P| may later change (set_budget) up to max_budget: sets and workspaces are sized for it
        self.max_budget = max(1, budget, max_budget or 0)
        self.kv = kv
        self.hq = num_q_heads
        self.block = block
        self.topk = topk
        self.budget = budget
        self.alpha, self.beta, self.gamma = (float(x) for x in ema)
        self.scale = float(scale) if scale is not None else kv.head_dim ** -0.5
        B, H, d = kv.batch, kv.num_kv_heads, kv.head_dim
        if score_mode not in bd.SCORE_MODES:
            raise ValueError(f"score_mode must be one of {sorted(bd.SCORE_MODES)}")
        self.score_mode = score_mode
        self.meta = bd.build_meta(kv, block) if score_mode == "quest" else bd.build_mean_meta(kv, block)
        self.nmax = bd.max_blocks(kv, block)
        self.scores = torch.zeros((B, H, self.nmax), dtype=torch.float64, device=dev)
        self.level = torch.zeros_like(self.scores)
        self.trend = torch.zeros_like(self.scores)
        self.live = torch.zeros((B, H), dtype=torch.int32, device=dev)
        # P (double-buffered) and M carry page work lists: the predictor writes P's physical pages a step
        # ahead and the top-K writes M's, so the speculative pass and repair start on K/V loads
        lb = block if page_lists else 0
        self.P = [bd.BlockSet.empty(B, H, self.max_budget, dev, lb), bd.BlockSet.empty(B, H, self.max_budget, dev, lb)]
        self.cur = 0
        self.A = bd.BlockSet.empty(B, H, max(1, topk), dev)
        self.M = bd.BlockSet.empty(B, H, max(1, topk), dev, lb)
        self.state = bd.AttnState.empty(B, num_q_heads, d, dev)
        self.out = torch.zeros((B, num_q_heads, d), dtype=torch.float32, device=dev)
        self.ws_spec = bd.select_spec_workspace_for(kv, num_q_heads, block, topk, self.max_budget)
        self.ws_select = bd.select_workspace_for(kv, block, topk, score_mode)   # separate selection (long rows)
        self.ws_repair = bd.workspace_for(kv, num_q_heads, block, max(1, topk))
        # the layer step in one launch (prr_layer_step), or select_spec then repair
        self.fused = bool(fused)
        self.ws_layer = (bd.layer_step_workspace_for(kv, num_q_heads, block, topk, self.max_budget, max(1, topk))
                         if self.fused else None)
        # the predictor's workspace depends on |P| and is not monotone in it (a budget with no part-parallel
        # plan needs none): sized for every budget set_budget may choose
        self.ws_predict = bd.predict_workspace_for(B, H, self.nmax, range(1, self.max_budget + 1), dev)
        self._streams = None
        self.pending_predict: Optional[bd.PredictArgs] = None

    def set_budget(self, budget: int):
        """|P| of the predictions made from the next step on (e.g. from speculation_budget() as the context
        grows); 0 <= budget <= max_budget (0: no speculation, repair covers all of A).  The set already
        predicted for the next step keeps its size."""
        if not 0 <= int(budget) <= self.max_budget:
            raise ValueError(f"budget {budget} outside [0, {self.max_budget}] (raise max_budget at construction)")
        self.budget = int(budget)

    @property
    def P_cur(self) -> bd.BlockSet:
        return self.P[self.cur]

    def append(self, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
        """Append one decoded token per sequence to the cache and fold it into this layer's metadata."""
        bd.append(self.kv, self.block, k_new, v_new, self.meta, mode=self.score_mode, stream=stream)

    def reset(self):
        """Forget the predictor state (a fresh decode: the first step runs with P empty)."""
        self.pending_predict = None
        if self._streams is not None:
            torch.cuda.current_stream().wait_event(self._streams[3])
        self.level.zero_()
        self.trend.zero_()
        self.live.zero_()
        for p in self.P:
            p.count.zero_()
        self.cur = 0

    def step(self, q: torch.Tensor, timers: Optional[StepTimers] = None, carry: Optional[bd.PredictArgs] = None,
             defer_predict: bool = False) -> torch.Tensor:
        """Enqueue one layer step for queries q [B][Hq][d] on the current stream; returns the normalised
        output tensor (valid once the stream reaches it).

        carry: another layer's pending predictor step, run by workgroups of this step's selection +
        speculative launch.  defer_predict: leave this step's predictor pending (``pending_predict``) for
        a later launch to carry; it must run before this layer's next step."""
        s = torch.cuda.current_stream()
        if self._streams is not None:
            s.wait_event(self._streams[3])   # a previous two-stream step's predictor
        if self.pending_predict is not None:
            raise RuntimeError("this layer's previous predictor step has not been run")
        P, Pn = self.P[self.cur], self.P[1 - self.cur]
        if timers and timers.start:
            timers.start.record(s)
        if self.fused:
            if timers and (timers.kernel_start or timers.kernel_end):
                bd.time_next_kernel(timers.kernel_start, timers.kernel_end)
            bd.layer_step(q, self.kv, self.meta, self.block, self.topk, P, self.scale, self.scores, self.A, self.M,
                          self.state, out=self.out, ws=self.ws_layer, mode=self.score_mode, pred=carry, stream=s)
            if timers and timers.select_spec_end:
                timers.select_spec_end.record(s)
        else:
            if timers and timers.kernel_start:
                bd.time_next_kernel(timers.kernel_start, None)
            bd.select_spec(q, self.kv, self.meta, self.block, self.topk, P, self.scale, scores=self.scores, A=self.A,
                           M=self.M, out=self.state, ws=self.ws_spec, mode=self.score_mode, pred=carry, stream=s)
            if timers and timers.select_spec_end:
                timers.select_spec_end.record(s)
            if timers and timers.kernel_end:
                bd.time_next_kernel(None, timers.kernel_end)
            bd.repair(q, self.kv, self.block, self.M, self.scale, self.state, out=self.out, ws=self.ws_repair,
                      stream=s)
        if timers and timers.repair_end:
            timers.repair_end.record(s)
        args = bd.PredictArgs(self.scores, self.kv.seq_len, self.block, self.alpha, self.beta, self.gamma,
                              self.budget, self.level, self.trend, self.live, Pn, self.ws_predict, self.kv)
        if defer_predict:
            self.pending_predict = args
        else:
            run_predict(args, s)
        if timers and timers.predict_end:
            timers.predict_end.record(s)
        self.cur = 1 - self.cur
        return self.out

    def take_pending_predict(self) -> Optional[bd.PredictArgs]:
        """Hand the deferred predictor step to the caller (who must enqueue it) and clear it."""
        args, self.pending_predict = self.pending_predict, None
        return args

    def step_two_streams(self, q: torch.Tensor, timers: Optional[TwoStreamTimers] = None) -> torch.Tensor:
        """The same step on three streams joined by events (the pages' schedule):
          critical:  wait(e_pred) -> record e_ready -> select -> record e_sel; wait(e_spec) -> repair
          side:      wait(e_ready) -> spec_attn(P) -> record e_spec
          predictor: wait(e_sel) -> predict -> record e_pred
        """
        crit = torch.cuda.current_stream()
        if self._streams is None:
            dev = self.kv.k.device
            e_pred = torch.cuda.Event()
            aux = torch.cuda.Stream(device=dev)
            e_pred.record(aux)
            self._streams = (torch.cuda.Stream(device=dev), aux, (torch.cuda.Event(), torch.cuda.Event(),
                                                                  torch.cuda.Event()), e_pred)
        side, aux, (e_ready, e_sel, e_spec), e_pred = self._streams
        P, Pn = self.P[self.cur], self.P[1 - self.cur]
        if timers and timers.start:
            timers.start.record(crit)
        crit.wait_event(e_pred)
        e_ready.record(crit)
        side.wait_event(e_ready)
        bd.select(q, self.kv, self.meta, self.block, self.topk, P=P, scores=self.scores, A=self.A, M=self.M,
                  mode=self.score_mode, stream=crit, ws=self.ws_select)
        e_sel.record(crit)
        if timers and timers.select_end:
            timers.select_end.record(crit)
        if timers and timers.spec_start:
            timers.spec_start.record(side)
        bd.spec_attn(q, self.kv, self.block, P, self.scale, out=self.state, ws=self.ws_spec, stream=side)
        if timers and timers.spec_end:
            timers.spec_end.record(side)
        e_spec.record(side)
        aux.wait_event(e_sel)
        bd.predict(self.scores, self.kv.seq_len, self.block, self.alpha, self.beta, self.gamma, self.budget,
                   self.level, self.trend, self.live, P_next=Pn, ws=self.ws_predict, stream=aux, kv=self.kv)
        e_pred.record(aux)
        crit.wait_event(e_spec)
        if timers and timers.repair_start:
            timers.repair_start.record(crit)
        bd.repair(q, self.kv, self.block, self.M, self.scale, self.state, out=self.out, ws=self.ws_repair,
                  stream=crit)
        if timers and timers.repair_end:
            timers.repair_end.record(crit)
        self.cur = 1 - self.cur
        return self.out


def run_predict(args: bd.PredictArgs, stream=None):
    """Enqueue a predictor step on its own."""
    bd.predict(args.scores, args.seq_len, args.block, args.alpha, args.beta, args.gamma, args.budget, args.level,
               args.trend, args.live, P_next=args.P_next, ws=args.ws, stream=stream, kv=args.kv)


class PRRStack:
    """The attention layers of a model through one decode step each, in order ([paper] §1 and the
    Figure 1 flow for each layer; [paper] §4.2: every layer has its own calibrated (alpha, beta, gamma)).

    Each layer keeps its own cache (and sequence lengths), metadata, predictor state and sets.  A layer's
    predictor needs only that layer's scores, so it is deferred and carried by the next layer's
    selection + speculative launch, whose spare workgroup slots absorb it; the last layer's rides in
    the first layer's launch of the next decode step.  ``flush`` runs a still-pending one on its own
    (before reading predictor state, or at the end of decoding).  Results equal running every layer's
    steps one after another."""

    def __init__(self, layers: list):
        self.layers = list(layers)
        self.pending: Optional[bd.PredictArgs] = None
        self.pending_owner = -1

    def step(self, qs, k_new=None, v_new=None, timers=None, before_layer=None) -> list:
        """One decode step through every layer: qs[l] [B][Hq][d]; k_new[l], v_new[l] [B][Hkv][d] (optional)
        are appended to layer l's cache first.  Returns each layer's output tensor.  timers[l]: optional
        StepTimers of layer l's step; before_layer(l): optional work enqueued before layer l (e.g. the
        rest of the model's layer)."""
        outs = []
        for i, layer in enumerate(self.layers):
            if self.pending_owner == i:
                # a layer's own predictor writes the set its next selection reads: it runs first, alone
                self.flush()
            if before_layer is not None:
                before_layer(i)
            if k_new is not None:
                layer.append(k_new[i], v_new[i])
            outs.append(layer.step(qs[i], timers[i] if timers else None, carry=self.pending, defer_predict=True))
            self.pending, self.pending_owner = layer.take_pending_predict(), i
        return outs

    def flush(self, stream=None):
        if self.pending is not None:
            run_predict(self.pending, stream)
        self.pending, self.pending_owner = None, -1

    def reset(self):
        self.pending, self.pending_owner = None, -1
        for layer in self.layers:
            layer.reset()


def speculation_budget(table: bd.BudgetTable, context: int, topk: int) -> int:
    """|P| in blocks for a layer at `context` tokens ([paper] §4.4; Eq. 1, |P| <= delta |A|): the library's
    choice (prr_budget_choose), floor(delta K) for the table's largest delta whose speculative pass ends no
    later than selection, or for its smallest delta when none fits."""
    return table.budget_blocks(float(context), int(topk))
