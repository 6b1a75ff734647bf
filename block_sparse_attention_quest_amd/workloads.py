"""Seeded synthetic inputs for the PRR decode hot path.

This module only *makes inputs*: queries, a paged K/V cache, page tables, sequence lengths, a prefill
score matrix, and (given an already-computed selected set) a speculative set with a prescribed overlap.
It holds none of the method's arithmetic (no scoring, no top-K, no attention, no EMA), so both the HIP
path and the CPU oracle can consume what it produces without sharing code.

Paged cache layout (the library's own format, see include/prr.h):
  k_cache [num_pages][num_kv_heads][page_size][head_dim]   token-major page tiles
  v_cache [num_pages][num_kv_heads][head_dim][page_size]   channel-major page tiles
  page_table [batch][max_pages] int32, logical page -> physical page
  seq_len [batch] int32

Workload shapes follow the pages' evaluation settings: GQA 32 query / 8 KV heads with head_dim 128 and
128K context (paper, §5.4 / Table 3), Llama-3-8B-shaped heads (paper, §5.1), block sizes 16-64 and token
budgets 1K-8K (paper, Table 3), about 68% adjacent-step overlap of the selected sets (paper, §2.2 /
Figure 3), and lognormal-like positive prefill scores for calibration (paper, §4.2).  Real benchmark
traces (LongBench, InfiniteBench, RULER, AIME, MATH500) are not available; these synthetic inputs stand
in for them.

Generation runs in torch on any device (CPU for small shapes, the GPU for the large ones).  bf16 values
are produced by round-to-nearest-even from fp32 samples; the oracle reads the exact stored bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np
import torch

PAGE_SIZE = 16

# Component ids used to derive independent seeds (seed * 64 + id).
_Q, _K, _V, _PLANT, _PERM, _CENTRE, _DRIFT, _PSET, _CALIB, _LEN, _APPK, _APPV = range(12)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype, selection budget and input structure knobs."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int              # tokens per sequence (all sequences unless seq_lens is given)
    block: int                # selection block size S in tokens (multiple of PAGE_SIZE)
    topk: int                 # budget K in blocks
    dtype: str                # "f32" or "bf16" (q, K and V share it), or "fp8" (E4M3 K and V, bf16 q)
    seed: int
    steps: int = 1            # decode steps with distinct queries
    shuffle_pages: bool = True
    seq_lens: Optional[Sequence[int]] = None   # ragged per-sequence lengths (override context)
    # speculative-set construction for single-step workloads: |P n A| and |P \ A|
    spec_hit: int = -1
    spec_miss: int = -1
    # planted heavy blocks: keys of `planted` blocks per (seq, kv head) get `plant_gain` * q_hat added,
    # q_hat = unit vector of the group's first query (step 0)
    planted: int = 0
    plant_gain: float = 8.0
    # multi-step query drift: q^t = mu + x^t, x^t = rho x^{t-1} + sqrt(1-rho^2) xi^t, mu = gain * N(0, I)
    drift_rho: float = 0.0
    query_mean_gain: float = 0.0
    # per-block key centres c_p ~ N(0, std^2 I) added to every key of the block
    block_centre_std: float = 0.0
    # EMA parameters (alpha, beta, gamma) used by multi-step workloads
    ema: tuple = (0.6, 0.3, 0.5)
    # prefill score matrix for calibration (rows x blocks); 0 = none
    calib_rows: int = 0
    calib_blocks: int = 0
    # decode-loop appends: tokens per sequence the cache has room for beyond the initial lengths
    append_tokens: int = 0

    # ---- derived sizes ----
    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def lengths(self) -> list:
        if self.seq_lens is not None:
            return [int(x) for x in self.seq_lens]
        return [self.context] * self.batch

    @property
    def max_pages(self) -> int:
        longest = max(self.lengths) + self.append_tokens
        # room for whole blocks so a block's pages always exist in the table
        nblk = -(-longest // self.block)
        return nblk * (self.block // PAGE_SIZE)

    @property
    def num_pages(self) -> int:
        return self.batch * self.max_pages

    @property
    def max_blocks(self) -> int:
        return self.max_pages * PAGE_SIZE // self.block

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def torch_dtype(self):
        """dtype of the K/V cache."""
        return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[self.dtype]

    @property
    def q_torch_dtype(self):
        """dtype of the queries (an fp8 cache is queried in bf16)."""
        return torch.bfloat16 if self.dtype == "fp8" else self.torch_dtype

    def blocks_of(self, b: int) -> int:
        return -(-self.lengths[b] // self.block)

    def kv_bytes_per_token(self) -> int:
        return 2 * self.head_dim * {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]


# The five configurations of the hot path (tiny parity case, Llama-3-8B layer, 128K x 64 steps,
# 512K paged, 70B-shaped share with calibration).
C1 = Workload("tiny", 1, 4, 1, 64, 1024, 16, 8, "f32", seed=1, shuffle_pages=False,
              spec_hit=5, spec_miss=3)
C2 = Workload("llama3_8b_32k", 1, 32, 8, 128, 32768, 16, 128, "bf16", seed=2,
              spec_hit=87, spec_miss=41, planted=32, plant_gain=8.0)
# query_mean_gain 0.64 puts the mean adjacent-step top-K overlap at ~0.68 (measured with the oracle's
# selection over all 8 kv heads and 64 steps); block_centre_std barely moves it.
C3 = Workload("ctx128k_b8_64steps", 8, 32, 8, 128, 131072, 64, 64, "bf16", seed=3, steps=64,
              drift_rho=0.9, query_mean_gain=0.64, block_centre_std=0.35, ema=(0.6, 0.3, 0.5))
C4 = Workload("ctx512k_paged", 1, 32, 8, 128, 524288, 16, 256, "bf16", seed=4,
              spec_hit=174, spec_miss=82)
C5 = Workload("llama70b_share_256k", 4, 64, 8, 128, 262144, 32, 128, "bf16", seed=5, steps=16,
              drift_rho=0.9, query_mean_gain=0.64, block_centre_std=0.35,
              calib_rows=8192, calib_blocks=512)

CONFIGS = {w.name: w for w in (C1, C2, C3, C4, C5)}


def scaled(w: Workload, **kw) -> Workload:
    """A copy of `w` with some fields replaced (used for reduced-size parity cases)."""
    return replace(w, **kw)


def _gen(w: Workload, comp: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(w.seed) * 64 + comp)
    return g


def _rng(w: Workload, comp: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(w.seed), comp]))


@dataclass
class Inputs:
    """Device- or host-resident inputs of one workload (torch tensors)."""

    w: Workload
    q: torch.Tensor            # [steps][B][Hq][d]
    k_cache: torch.Tensor      # [num_pages][Hkv][16][d]
    v_cache: torch.Tensor      # [num_pages][Hkv][d][16]
    page_table: torch.Tensor   # [B][max_pages] int32
    seq_len: torch.Tensor      # [B] int32
    planted: Optional[torch.Tensor] = None   # [B][Hkv][planted] int64 logical block ids
    extras: dict = field(default_factory=dict)


def make_page_table(w: Workload) -> torch.Tensor:
    """Logical -> physical page map; a random permutation of all pages when shuffle_pages."""
    n = w.num_pages
    if w.shuffle_pages:
        perm = _rng(w, _PERM).permutation(n)
    else:
        perm = np.arange(n)
    return torch.from_numpy(perm.reshape(w.batch, w.max_pages).astype(np.int32))


def make_queries(w: Workload, device="cpu") -> torch.Tensor:
    """Queries for every decode step, [steps][B][Hq][d] in the workload dtype."""
    g = _gen(w, _Q, device)
    shape = (w.batch, w.num_q_heads, w.head_dim)
    if w.steps == 1 or w.drift_rho == 0.0:
        q = torch.randn((w.steps,) + shape, generator=g, device=device, dtype=torch.float32)
    else:
        mu = w.query_mean_gain * torch.randn(shape, generator=g, device=device)
        x = torch.randn(shape, generator=g, device=device)
        innov = math.sqrt(1.0 - w.drift_rho ** 2)
        qs = []
        for _ in range(w.steps):
            qs.append(mu + x)
            x = w.drift_rho * x + innov * torch.randn(shape, generator=g, device=device)
        q = torch.stack(qs)
    return q.to(w.q_torch_dtype)


def _block_pages(w: Workload, page_table: torch.Tensor, b: int, blocks: torch.Tensor) -> torch.Tensor:
    """Physical pages of the given logical blocks of sequence b, [n][block/16]."""
    ppb = w.block // PAGE_SIZE
    lp = blocks.view(-1, 1) * ppb + torch.arange(ppb, device=blocks.device).view(1, -1)
    return page_table[b].to(blocks.device)[lp].long()


def make_inputs(w: Workload, device="cpu") -> Inputs:
    """Generate q, the paged K/V cache, page table and lengths for workload w on `device`."""
    page_table = make_page_table(w).to(device)
    seq_len = torch.tensor(w.lengths, dtype=torch.int32, device=device)
    q = make_queries(w, device)
    shape_k = (w.num_pages, w.num_kv_heads, PAGE_SIZE, w.head_dim)
    gk = _gen(w, _K, device)
    k = torch.randn(shape_k, generator=gk, device=device, dtype=torch.float32)
    planted = None
    if w.block_centre_std > 0.0:
        gc = _gen(w, _CENTRE, device)
        for b in range(w.batch):
            nb = w.blocks_of(b)
            blocks = torch.arange(nb, device=device)
            pages = _block_pages(w, page_table, b, blocks)          # [nb][ppb]
            c = w.block_centre_std * torch.randn((nb, w.num_kv_heads, w.head_dim), generator=gc,
                                                 device=device)
            # k[page, kvh, t, :] += c[block, kvh, :]
            k[pages.reshape(-1)] += c.repeat_interleave(pages.shape[1], dim=0)[:, :, None, :]
    if w.planted > 0:
        rng = _rng(w, _PLANT)
        planted = torch.zeros((w.batch, w.num_kv_heads, w.planted), dtype=torch.int64)
        qf = q[0].float()
        for b in range(w.batch):
            nb = w.blocks_of(b)
            for h in range(w.num_kv_heads):
                ids = np.sort(rng.choice(nb, size=w.planted, replace=False))
                planted[b, h] = torch.from_numpy(ids)
                u = qf[b, h * w.group]
                u = u / torch.linalg.vector_norm(u)
                pages = _block_pages(w, page_table, b, torch.from_numpy(ids).to(device))
                k[pages.reshape(-1), h] += w.plant_gain * u
    k_cache = to_cache_dtype(k, w)
    del k
    gv = _gen(w, _V, device)
    v_cache = to_cache_dtype(torch.randn((w.num_pages, w.num_kv_heads, w.head_dim, PAGE_SIZE), generator=gv,
                                         device=device, dtype=torch.float32), w)
    return Inputs(w, q, k_cache, v_cache, page_table, seq_len, planted)


def make_append_tokens(w: Workload, device="cpu"):
    """Keys and values of the decode-loop appends, [append_tokens][B][Hkv][d] each, N(0, 1) in the
    workload dtype."""
    shape = (w.append_tokens, w.batch, w.num_kv_heads, w.head_dim)
    k = torch.randn(shape, generator=_gen(w, _APPK, device), device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=_gen(w, _APPV, device), device=device, dtype=torch.float32)
    return to_cache_dtype(k, w), to_cache_dtype(v, w)


def to_cache_dtype(x: torch.Tensor, w: Workload) -> torch.Tensor:
    """Round generated fp32 values to the cache dtype (fp8: clamped to E4M3's finite range first)."""
    if w.dtype == "fp8":
        x = x.clamp(-448.0, 448.0)
    return x.to(w.torch_dtype)


def make_spec_set(w: Workload, selected: np.ndarray, n_blocks: int, n_hit: int, n_miss: int,
                  salt: int = 0) -> np.ndarray:
    """A speculative set with n_hit members of `selected` and n_miss non-members, in shuffled order.

    `selected` is an already-computed selected set (from whichever side); this function only samples.
    """
    rng = np.random.default_rng(np.random.SeedSequence([int(w.seed), _PSET, int(salt)]))
    sel = np.asarray(selected, dtype=np.int64)
    others = np.setdiff1d(np.arange(n_blocks), sel)
    n_hit = min(n_hit, sel.size)
    n_miss = min(n_miss, others.size)
    hit = rng.choice(sel, size=n_hit, replace=False) if n_hit else np.zeros(0, np.int64)
    miss = rng.choice(others, size=n_miss, replace=False) if n_miss else np.zeros(0, np.int64)
    p = np.concatenate([hit, miss])
    rng.shuffle(p)
    return p.astype(np.int32)


def make_calibration_scores(w: Workload, rows: Optional[int] = None,
                            blocks: Optional[int] = None) -> np.ndarray:
    """Prefill score matrix IS[rows][blocks] (fp32): exp(mu_b + x_{phi,b}), mu_b ~ N(0,1), and x an
    AR(1) in phi with rho 0.9 and stationary std 0.5 - positive, lognormal marginals, temporally
    correlated rows so the predictor parameters matter."""
    rows = rows or w.calib_rows
    blocks = blocks or w.calib_blocks
    rng = _rng(w, _CALIB)
    rho, sd = 0.9, 0.5
    mu = rng.standard_normal(blocks)
    x = sd * rng.standard_normal(blocks)
    out = np.empty((rows, blocks), dtype=np.float64)
    innov = sd * math.sqrt(1.0 - rho * rho)
    for r in range(rows):
        out[r] = mu + x
        x = rho * x + innov * rng.standard_normal(blocks)
    return np.exp(out).astype(np.float32)


def ragged_lengths(w: Workload, lo: int, hi: int, salt: int = 0) -> list:
    """Per-sequence lengths drawn uniformly from [lo, hi] (for ragged parity cases)."""
    rng = np.random.default_rng(np.random.SeedSequence([int(w.seed), _LEN, int(salt)]))
    return [int(x) for x in rng.integers(lo, hi + 1, size=w.batch)]


# ---- host views used by both sides (layout decoding only, no arithmetic of the method) ----

def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy; bf16 tensors come back as their raw uint16 bit patterns, fp8 tensors as their uint8
    codes."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()
