"""ctypes binding of libprr.so (argument marshalling only; every step runs in the HIP library).

Torch provides device memory and streams.  The functions here take torch tensors that already live on
the GPU, pass their device pointers and the current (or given) torch stream to the C entry points
declared in include/prr.h, and raise PrrError on a non-zero status.  There is no CPU fallback: if the
library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libprr.so")

PRR_F32, PRR_BF16, PRR_FP8 = 0, 1, 2
PAGE_SIZE = 16

# Every symbol include/prr.h declares.
EXPORTS = (
    "prr_max_blocks", "prr_meta_stride", "prr_meta_bytes", "prr_attn_workspace_bytes",
    "prr_workspace_clear", "prr_build_meta", "prr_mean_meta_bytes", "prr_build_mean_meta", "prr_append",
    "prr_select_workspace_bytes", "prr_select", "prr_select_spec_workspace_bytes", "prr_select_spec", "prr_select_spec_predict",
    "prr_layer_step_workspace_bytes", "prr_layer_step", "prr_predict_workspace_bytes",
    "prr_predict",
    "prr_spec_attn", "prr_spec_attn_noalloc",
    "prr_repair", "prr_calibrate_workspace_bytes", "prr_calibrate", "prr_budget_fit", "prr_budget_choose",
    "prr_time_next_kernel", "prr_strerror",
)


class PrrError(RuntimeError):
    def __init__(self, status: int, where: str, text: str):
        super().__init__(f"{where}: {text} (status {status})")
        self.status = status


class KvCacheStruct(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p), ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("dtype", ctypes.c_int)]


class BlockSetStruct(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("count", ctypes.c_void_p), ("cap", ctypes.c_int32),
                ("pages", ctypes.c_void_p)]


class AttnStateStruct(ctypes.Structure):
    _fields_ = [("acc", ctypes.c_void_p), ("l", ctypes.c_void_p), ("m", ctypes.c_void_p)]


class PredictArgsStruct(ctypes.Structure):
    _fields_ = [("scores", ctypes.c_void_p), ("seq_len", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("block", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("alpha", ctypes.c_double), ("beta", ctypes.c_double), ("gamma", ctypes.c_double),
                ("budget", ctypes.c_int32), ("level", ctypes.c_void_p), ("trend", ctypes.c_void_p),
                ("live", ctypes.c_void_p), ("P_next", ctypes.POINTER(BlockSetStruct)), ("ws", ctypes.c_void_p),
                ("ws_bytes", ctypes.c_size_t), ("kv", ctypes.POINTER(KvCacheStruct))]


_P = ctypes.POINTER
_VP, _I32, _SZ, _D, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double, ctypes.c_float

_SIGS = {
    "prr_max_blocks": (_I32, [_P(KvCacheStruct), _I32]),
    "prr_meta_stride": (_I32, [_P(KvCacheStruct), _I32]),
    "prr_meta_bytes": (_SZ, [_P(KvCacheStruct), _I32]),
    "prr_attn_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "prr_workspace_clear": (ctypes.c_int, [_VP, _SZ, _VP]),
    "prr_build_meta": (ctypes.c_int, [_P(KvCacheStruct), _I32, _VP, _VP]),
    "prr_mean_meta_bytes": (_SZ, [_P(KvCacheStruct), _I32]),
    "prr_build_mean_meta": (ctypes.c_int, [_P(KvCacheStruct), _I32, _VP, _VP]),
    "prr_append": (ctypes.c_int, [_P(KvCacheStruct), _I32, _VP, _VP, _VP, ctypes.c_int, _VP, _VP]),
    "prr_select_workspace_bytes": (_SZ, [_P(KvCacheStruct), ctypes.c_int, _I32, _I32]),
    "prr_select": (ctypes.c_int, [_VP, _I32, _P(KvCacheStruct), _VP, ctypes.c_int, _I32, _I32,
                                  _P(BlockSetStruct), _VP, _P(BlockSetStruct), _P(BlockSetStruct), _VP, _SZ,
                                  _VP]),
    "prr_select_spec_workspace_bytes": (_SZ, [_P(KvCacheStruct), _I32, _I32, _I32, _I32]),
    "prr_select_spec": (ctypes.c_int, [_VP, _I32, _P(KvCacheStruct), _VP, ctypes.c_int, _I32, _I32,
                                       _P(BlockSetStruct), _VP, _P(BlockSetStruct), _P(BlockSetStruct), _F,
                                       _P(AttnStateStruct), _VP, _SZ, _VP]),
    "prr_select_spec_predict": (ctypes.c_int, [_VP, _I32, _P(KvCacheStruct), _VP, ctypes.c_int, _I32, _I32,
                                               _P(BlockSetStruct), _VP, _P(BlockSetStruct), _P(BlockSetStruct),
                                               _F, _P(AttnStateStruct), _VP, _SZ, _P(PredictArgsStruct), _VP]),
    "prr_layer_step_workspace_bytes": (_SZ, [_P(KvCacheStruct), _I32, _I32, _I32, _I32, _I32]),
    "prr_layer_step": (ctypes.c_int, [_VP, _I32, _P(KvCacheStruct), _VP, ctypes.c_int, _I32, _I32, _P(BlockSetStruct),
                                      _VP, _P(BlockSetStruct), _P(BlockSetStruct), _F, _P(AttnStateStruct), _VP, _VP,
                                      _SZ, _P(PredictArgsStruct), _VP]),
    "prr_predict_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "prr_predict": (ctypes.c_int, [_VP, _VP, _I32, _I32, _I32, _I32, _D, _D, _D, _I32, _VP, _VP, _VP,
                                   _P(BlockSetStruct), _P(KvCacheStruct), _VP, _SZ, _VP]),
    "prr_spec_attn": (ctypes.c_int, [_VP, _I32, _P(KvCacheStruct), _I32, _P(BlockSetStruct), _F,
                                     _P(AttnStateStruct), _VP, _SZ, _VP]),
    "prr_spec_attn_noalloc": (ctypes.c_int, [_VP, _I32, _P(KvCacheStruct), _I32, _P(BlockSetStruct), _F,
                                             _P(AttnStateStruct), _VP]),
    "prr_repair": (ctypes.c_int, [_VP, _I32, _P(KvCacheStruct), _I32, _P(BlockSetStruct), _F,
                                  _P(AttnStateStruct), _VP, _VP, _SZ, _VP]),
    "prr_calibrate_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "prr_calibrate": (ctypes.c_int, [_VP, _I32, _I32, _I32, _VP, _I32, _VP, _VP, _VP, _SZ, _VP]),
    "prr_budget_fit": (ctypes.c_int, [_VP, _I32, _VP, _VP, _I32, _VP, _I32, _VP]),
    "prr_budget_choose": (ctypes.c_int, [_VP, _I32, _VP, _VP, _I32, _VP, _I32, _VP, _D, _VP, _VP, _I32, _VP]),
    "prr_time_next_kernel": (ctypes.c_int, [_VP, _VP]),
    "prr_strerror": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None

# prr_score_mode: how selection scores a block (Quest's min/max bound, or the block's mean key)
SCORE_MODES = {"quest": 0, "mean": 1}


def _mode(mode: str) -> int:
    if mode not in SCORE_MODES:
        raise ValueError(f"score mode must be one of {sorted(SCORE_MODES)}, not {mode!r}")
    return SCORE_MODES[mode]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libprr.so and declare its signatures.  Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libprr.so not found at {path}; build it with "
                          "`python -m block_sparse_attention_quest_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        raise PrrError(status, where, load_library().prr_strerror(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PRR_BF16
    if t.dtype == torch.float32:
        return PRR_F32
    if t.dtype == torch.float8_e4m3fn:
        return PRR_FP8
    raise TypeError(f"unsupported dtype {t.dtype}")


# --------------------------------------------------------------------------------------------------
# Tensor-level containers
# --------------------------------------------------------------------------------------------------


@dataclass
class KVCache:
    """Paged cache on the device: k [pages][Hkv][16][d], v [pages][Hkv][d][16], page_table [B][P],
    seq_len [B]."""

    k: torch.Tensor
    v: torch.Tensor
    page_table: torch.Tensor
    seq_len: torch.Tensor

    @property
    def batch(self) -> int:
        return self.page_table.shape[0]

    @property
    def num_kv_heads(self) -> int:
        return self.k.shape[1]

    @property
    def head_dim(self) -> int:
        return self.k.shape[3]

    def struct(self) -> KvCacheStruct:
        return KvCacheStruct(self.k.data_ptr(), self.v.data_ptr(), self.page_table.data_ptr(),
                             self.seq_len.data_ptr(), self.batch, self.num_kv_heads, self.head_dim,
                             self.k.shape[2], self.k.shape[0], self.page_table.shape[1],
                             _dtype_code(self.k))


@dataclass
class BlockSet:
    """idx [B][Hkv][cap] int32, count [B][Hkv] int32 (device); pages (optional) [B][Hkv][cap * block / 16]
    int32: the set's page work list (physical page of every page of the set's blocks, -1 for a page with no
    token yet), written by the call that produces the set and read by the attention passes over it."""

    idx: torch.Tensor
    count: torch.Tensor
    pages: Optional[torch.Tensor] = None

    @property
    def cap(self) -> int:
        return self.idx.shape[-1]

    @staticmethod
    def empty(batch: int, hkv: int, cap: int, device="cuda", block: int = 0) -> "BlockSet":
        """block > 0: with a page work list for that block size."""
        pages = (torch.full((batch, hkv, cap * (block // PAGE_SIZE)), -1, dtype=torch.int32, device=device)
                 if block > 0 else None)
        return BlockSet(torch.zeros((batch, hkv, cap), dtype=torch.int32, device=device),
                        torch.zeros((batch, hkv), dtype=torch.int32, device=device), pages)

    def struct(self) -> BlockSetStruct:
        return BlockSetStruct(self.idx.data_ptr(), self.count.data_ptr(), self.cap,
                              self.pages.data_ptr() if self.pages is not None else None)

    def lists(self):
        """Host copy as nested python lists [b][kvh] -> list of block ids."""
        idx = self.idx.cpu().numpy()
        cnt = self.count.cpu().numpy()
        return [[idx[b, h, :cnt[b, h]].tolist() for h in range(idx.shape[1])] for b in range(idx.shape[0])]


@dataclass
class AttnState:
    """acc [B][Hq][d] (unnormalised), l [B][Hq], m [B][Hq] (natural log units), fp32 device."""

    acc: torch.Tensor
    l: torch.Tensor
    m: torch.Tensor

    @staticmethod
    def empty(batch: int, hq: int, d: int, device="cuda") -> "AttnState":
        return AttnState(torch.zeros((batch, hq, d), dtype=torch.float32, device=device),
                         torch.zeros((batch, hq), dtype=torch.float32, device=device),
                         torch.full((batch, hq), float("-inf"), dtype=torch.float32, device=device))

    def clone(self) -> "AttnState":
        return AttnState(self.acc.clone(), self.l.clone(), self.m.clone())

    def struct(self) -> AttnStateStruct:
        return AttnStateStruct(self.acc.data_ptr(), self.l.data_ptr(), self.m.data_ptr())


class Workspace:
    """A zero-initialised device buffer for one stream's attention calls."""

    def __init__(self, nbytes: int, device="cuda"):
        self.buf = torch.zeros(max(256, int(nbytes)), dtype=torch.uint8, device=device)

    @property
    def nbytes(self) -> int:
        return self.buf.numel()

    def ptr(self):
        return ctypes.c_void_p(self.buf.data_ptr())


# --------------------------------------------------------------------------------------------------
# Entry points
# --------------------------------------------------------------------------------------------------


def _event_handle(ev) -> Optional[ctypes.c_void_p]:
    if ev is None:
        return None
    if not ev.cuda_event:   # torch creates the HIP event at its first record
        ev.record()
    return ctypes.c_void_p(ev.cuda_event)


def time_next_kernel(start, stop):
    """Arm two torch.cuda.Event(enable_timing=True) events (either may be None) for the next library call
    on this thread that enqueues GPU work: start takes the start of its first kernel and stop the end of
    its last, so start.elapsed_time(stop) is the GPU time of the call's kernels (prr_time_next_kernel)."""
    _check(load_library().prr_time_next_kernel(_event_handle(start), _event_handle(stop)), "prr_time_next_kernel")


def max_blocks(kv: KVCache, block: int) -> int:
    s = kv.struct()
    return load_library().prr_max_blocks(ctypes.byref(s), block)


def meta_stride(kv: KVCache, block: int) -> int:
    s = kv.struct()
    return load_library().prr_meta_stride(ctypes.byref(s), block)


def attn_workspace_bytes(batch: int, hq: int, hkv: int, d: int, block: int, cap: int) -> int:
    return load_library().prr_attn_workspace_bytes(batch, hq, hkv, d, block, cap)


def workspace_for(kv: KVCache, hq: int, block: int, cap: int) -> Workspace:
    return Workspace(attn_workspace_bytes(kv.batch, hq, kv.num_kv_heads, kv.head_dim, block, cap),
                     device=kv.k.device)


def select_spec_workspace_for(kv: KVCache, hq: int, block: int, topk: int, cap: int) -> Workspace:
    """Workspace for prr_select_spec (attention workspace plus top-K candidates)."""
    s = kv.struct()
    return Workspace(load_library().prr_select_spec_workspace_bytes(ctypes.byref(s), hq, block, topk, cap),
                     kv.k.device)


def predict_workspace_for(batch: int, num_kv_heads: int, max_blocks: int, budget, device="cuda"):
    """Workspace for predict() at |P| = budget, or at every budget of an iterable of them (the largest
    size any of them needs); None where none needs one (short rows)."""
    lib = load_library()
    budgets = [budget] if isinstance(budget, int) else list(budget)
    n = max((lib.prr_predict_workspace_bytes(batch, num_kv_heads, max_blocks, b) for b in budgets), default=0)
    return Workspace(n, device) if n else None


def workspace_clear(ws: Workspace, stream=None):
    _check(load_library().prr_workspace_clear(ws.ptr(), ws.nbytes, _stream(stream)), "prr_workspace_clear")


def build_meta(kv: KVCache, block: int, meta: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Block min/max metadata [B][Hkv][d][2][stride] in the cache dtype (bf16 for an fp8 cache)."""
    lib = load_library()
    s = kv.struct()
    if meta is None:
        stride = lib.prr_meta_stride(ctypes.byref(s), block)
        dt = torch.bfloat16 if kv.k.dtype == torch.float8_e4m3fn else kv.k.dtype
        meta = torch.empty((kv.batch, kv.num_kv_heads, kv.head_dim, 2, stride), dtype=dt, device=kv.k.device)
    _check(lib.prr_build_meta(ctypes.byref(s), block, _ptr(meta), _stream(stream)), "prr_build_meta")
    return meta


def build_mean_meta(kv: KVCache, block: int, meta: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Mean-pooled block metadata [B][Hkv][d][stride] fp32 (the channel-wise mean key of every block)."""
    lib = load_library()
    s = kv.struct()
    if meta is None:
        stride = lib.prr_meta_stride(ctypes.byref(s), block)
        meta = torch.empty((kv.batch, kv.num_kv_heads, kv.head_dim, stride), dtype=torch.float32,
                           device=kv.k.device)
    _check(lib.prr_build_mean_meta(ctypes.byref(s), block, _ptr(meta), _stream(stream)), "prr_build_mean_meta")
    return meta


def append(kv: KVCache, block: int, k_new: torch.Tensor, v_new: torch.Tensor, meta: torch.Tensor,
           mode: str = "quest", stream=None):
    """Append one token per sequence (k_new, v_new: [B][Hkv][d]) to the paged cache at position seq_len,
    fold its key into the metadata of its block (min/max for mode "quest", the block mean for "mean"),
    and advance kv.seq_len in place."""
    lib = load_library()
    s = kv.struct()
    _check(lib.prr_append(ctypes.byref(s), block, _ptr(k_new), _ptr(v_new), _ptr(meta), _mode(mode),
                          _ptr(kv.seq_len), _stream(stream)), "prr_append")


def select_workspace_for(kv: KVCache, block: int, topk: int, mode: str = "quest") -> Optional[Workspace]:
    """Workspace of prr_select (zeroed), or None where it would not be used (rows of up to 8192 blocks).
    With it, longer rows are ranked in part-parallel stages; rows above 32768 blocks need it."""
    s = kv.struct()
    n = load_library().prr_select_workspace_bytes(ctypes.byref(s), _mode(mode), block, topk)
    return Workspace(n, kv.k.device) if n else None


def select(q: torch.Tensor, kv: KVCache, meta: torch.Tensor, block: int, topk: int,
           P: Optional[BlockSet] = None, scores: Optional[torch.Tensor] = None,
           A: Optional[BlockSet] = None, M: Optional[BlockSet] = None, mode: str = "quest", stream=None,
           ws: Optional[Workspace] = None, staged: bool = True):
    """Block scores [B][Hkv][Nmax] fp64 (Quest's bound, or the mean key's product for mode "mean"),
    A (top-k, ascending) and M = A \\ P when P is given.  ws: select_workspace_for (allocated here when
    none is given and staged is true: rows above 8192 blocks are then ranked in part-parallel stages;
    staged false and no ws: one top-K workgroup per row, up to 32768 blocks)."""
    lib = load_library()
    if ws is None and staged:
        ws = select_workspace_for(kv, block, topk, mode)
    s = kv.struct()
    nmax = lib.prr_max_blocks(ctypes.byref(s), block)
    B, H = kv.batch, kv.num_kv_heads
    dev = kv.k.device
    if scores is None:
        scores = torch.zeros((B, H, nmax), dtype=torch.float64, device=dev)
    if A is None:
        A = BlockSet.empty(B, H, max(1, topk), dev)
    if P is not None and M is None:
        M = BlockSet.empty(B, H, max(1, topk), dev)
    a_s = A.struct()
    p_s = P.struct() if P is not None else None
    m_s = M.struct() if M is not None else None
    st = lib.prr_select(_ptr(q), q.shape[1], ctypes.byref(s), _ptr(meta), _mode(mode), block, topk,
                        ctypes.byref(p_s) if p_s is not None else None, _ptr(scores), ctypes.byref(a_s),
                        ctypes.byref(m_s) if m_s is not None else None, ws.ptr() if ws is not None else None,
                        ws.nbytes if ws is not None else 0, _stream(stream))
    _check(st, "prr_select")
    return scores, A, M


def select_spec(q: torch.Tensor, kv: KVCache, meta: torch.Tensor, block: int, topk: int, P: BlockSet,
                scale: float, scores: Optional[torch.Tensor] = None, A: Optional[BlockSet] = None,
                M: Optional[BlockSet] = None, out: Optional[AttnState] = None, ws: Optional[Workspace] = None,
                mode: str = "quest", pred: Optional["PredictArgs"] = None, stream=None):
    """select(q, ..., P) and spec_attn(q, ..., P) as one launch; returns (scores, A, M, state).  pred: a
    predictor step over other buffers (typically the previous layer's) carried by the same launch."""
    lib = load_library()
    s = kv.struct()
    nmax = lib.prr_max_blocks(ctypes.byref(s), block)
    B, Hq, d = q.shape
    H = kv.num_kv_heads
    dev = kv.k.device
    if scores is None:
        scores = torch.zeros((B, H, nmax), dtype=torch.float64, device=dev)
    if A is None:
        A = BlockSet.empty(B, H, max(1, topk), dev)
    if M is None:
        M = BlockSet.empty(B, H, max(1, topk), dev)
    if out is None:
        out = AttnState.empty(B, Hq, d, dev)
    if ws is None:
        ws = select_spec_workspace_for(kv, Hq, block, topk, P.cap)
    a_s, p_s, m_s, o_s = A.struct(), P.struct(), M.struct(), out.struct()
    if pred is None:
        st = lib.prr_select_spec(_ptr(q), Hq, ctypes.byref(s), _ptr(meta), _mode(mode), block, topk,
                                 ctypes.byref(p_s), _ptr(scores), ctypes.byref(a_s), ctypes.byref(m_s), float(scale),
                                 ctypes.byref(o_s), ws.ptr(), ws.nbytes, _stream(stream))
        _check(st, "prr_select_spec")
    else:
        pa, keep = pred.structs()
        st = lib.prr_select_spec_predict(_ptr(q), Hq, ctypes.byref(s), _ptr(meta), _mode(mode), block, topk,
                                         ctypes.byref(p_s), _ptr(scores), ctypes.byref(a_s), ctypes.byref(m_s),
                                         float(scale), ctypes.byref(o_s), ws.ptr(), ws.nbytes, ctypes.byref(pa),
                                         _stream(stream))
        _check(st, "prr_select_spec_predict")
    return scores, A, M, out


def layer_step_workspace_for(kv: KVCache, hq: int, block: int, topk: int, p_cap: int, m_cap: int) -> Workspace:
    """Workspace for layer_step() (prr_layer_step_workspace_bytes)."""
    s = kv.struct()
    return Workspace(load_library().prr_layer_step_workspace_bytes(ctypes.byref(s), hq, block, topk, p_cap, m_cap),
                     kv.k.device)


def layer_step(q: torch.Tensor, kv: KVCache, meta: torch.Tensor, block: int, topk: int, P: BlockSet, scale: float,
               scores: torch.Tensor, A: BlockSet, M: BlockSet, state: AttnState, out: Optional[torch.Tensor] = None,
               ws: Optional[Workspace] = None, mode: str = "quest", pred: Optional["PredictArgs"] = None, stream=None):
    """The layer step (prr_layer_step): selection (scores, A, M = A \\ P), the speculative pass over P and
    repair over M, the final state over P u M in `state` and acc / l in `out` (optional); one launch where
    the top-K finishes inside it.  pred: another layer's predictor step carried by the launch."""
    lib = load_library()
    Hq = q.shape[1]
    if ws is None:
        ws = layer_step_workspace_for(kv, Hq, block, topk, P.cap, M.cap)
    s = kv.struct()
    a_s, p_s, m_s, o_s = A.struct(), P.struct(), M.struct(), state.struct()
    pa = None
    if pred is not None:
        pa, keep = pred.structs()
    st = lib.prr_layer_step(_ptr(q), Hq, ctypes.byref(s), _ptr(meta), _mode(mode), block, topk, ctypes.byref(p_s),
                            _ptr(scores), ctypes.byref(a_s), ctypes.byref(m_s), float(scale), ctypes.byref(o_s),
                            _ptr(out), ws.ptr(), ws.nbytes, ctypes.byref(pa) if pa is not None else None,
                            _stream(stream))
    _check(st, "prr_layer_step")
    return state


@dataclass
class PredictArgs:
    """One predictor step's operands (those of predict()), to be carried by a select_spec launch."""

    scores: torch.Tensor
    seq_len: torch.Tensor
    block: int
    alpha: float
    beta: float
    gamma: float
    budget: int
    level: torch.Tensor
    trend: torch.Tensor
    live: torch.Tensor
    P_next: "BlockSet"
    ws: Optional["Workspace"] = None
    kv: Optional["KVCache"] = None   # needed when P_next has a page list (its page table)

    def struct(self, p_next_struct, kv_struct=None) -> PredictArgsStruct:
        """p_next_struct / kv_struct: the caller keeps them alive for the call."""
        B, H, nmax = self.scores.shape
        return PredictArgsStruct(_ptr(self.scores), _ptr(self.seq_len), B, H, self.block, nmax, float(self.alpha),
                                 float(self.beta), float(self.gamma), self.budget, _ptr(self.level),
                                 _ptr(self.trend), _ptr(self.live), ctypes.pointer(p_next_struct),
                                 self.ws.ptr() if self.ws is not None else None,
                                 self.ws.nbytes if self.ws is not None else 0,
                                 ctypes.pointer(kv_struct) if kv_struct is not None else None)

    def structs(self):
        """(args, keep-alive) for a call that carries this step."""
        pn = self.P_next.struct()
        ks = self.kv.struct() if self.kv is not None else None
        return self.struct(pn, ks), (pn, ks)


def predict(scores: torch.Tensor, seq_len: torch.Tensor, block: int, alpha: float, beta: float,
            gamma: float, budget: int, level: torch.Tensor, trend: torch.Tensor, live: torch.Tensor,
            P_next: Optional[BlockSet] = None, ws: Optional[Workspace] = None, stream=None,
            kv: Optional["KVCache"] = None) -> BlockSet:
    """One EMA step over scores [B][Hkv][Nmax]; updates level/trend/live in place; returns P_next.  ws
    (predict_workspace_for): long rows are then updated in parallel parts.  kv: the cache whose page table
    P_next's page list (if it has one) maps through."""
    lib = load_library()
    B, H, nmax = scores.shape
    if P_next is None:
        P_next = BlockSet.empty(B, H, max(1, budget), scores.device)
    ps = P_next.struct()
    ks = kv.struct() if kv is not None else None
    st = lib.prr_predict(_ptr(scores), _ptr(seq_len), B, H, block, nmax, float(alpha), float(beta),
                         float(gamma), budget, _ptr(level), _ptr(trend), _ptr(live), ctypes.byref(ps),
                         ctypes.byref(ks) if ks is not None else None,
                         ws.ptr() if ws is not None else None, ws.nbytes if ws is not None else 0,
                         _stream(stream))
    _check(st, "prr_predict")
    return P_next


def spec_attn(q: torch.Tensor, kv: KVCache, block: int, P: BlockSet, scale: float,
              out: Optional[AttnState] = None, ws: Optional[Workspace] = None, stream=None) -> AttnState:
    """Speculative attention over P: the unnormalised state (acc, l, m) of every query head."""
    lib = load_library()
    B, Hq, d = q.shape
    if out is None:
        out = AttnState.empty(B, Hq, d, q.device)
    if ws is None:
        ws = workspace_for(kv, Hq, block, P.cap)
    s, ps, os_ = kv.struct(), P.struct(), out.struct()
    st = lib.prr_spec_attn(_ptr(q), Hq, ctypes.byref(s), block, ctypes.byref(ps), float(scale),
                           ctypes.byref(os_), ws.ptr(), ws.nbytes, _stream(stream))
    _check(st, "prr_spec_attn")
    return out


def spec_attn_noalloc(q: torch.Tensor, kv: KVCache, block: int, P: BlockSet, scale: float,
                      out: Optional[AttnState] = None, stream=None) -> AttnState:
    """spec_attn with the library's own per-GPU buffer as workspace (prr_spec_attn_noalloc): no
    workspace argument, nothing allocated by the call; calls that overlap on one GPU race."""
    lib = load_library()
    B, Hq, d = q.shape
    if out is None:
        out = AttnState.empty(B, Hq, d, q.device)
    s, ps, os_ = kv.struct(), P.struct(), out.struct()
    st = lib.prr_spec_attn_noalloc(_ptr(q), Hq, ctypes.byref(s), block, ctypes.byref(ps), float(scale),
                                   ctypes.byref(os_), _stream(stream))
    _check(st, "prr_spec_attn_noalloc")
    return out


def repair(q: torch.Tensor, kv: KVCache, block: int, M: BlockSet, scale: float, state: AttnState,
           out: Optional[torch.Tensor] = None, ws: Optional[Workspace] = None, stream=None) -> AttnState:
    """Fold the missed blocks M into `state` in place; optionally write the normalised output."""
    lib = load_library()
    B, Hq, d = q.shape
    if ws is None:
        ws = workspace_for(kv, Hq, block, M.cap)
    s, ms, ss = kv.struct(), M.struct(), state.struct()
    st = lib.prr_repair(_ptr(q), Hq, ctypes.byref(s), block, ctypes.byref(ms), float(scale),
                        ctypes.byref(ss), _ptr(out), ws.ptr(), ws.nbytes, _stream(stream))
    _check(st, "prr_repair")
    return state


def calibration_grid(device="cuda") -> torch.Tensor:
    """The 80 candidates (alpha, beta, gamma) of the online calibration, alpha-major: alpha in
    {0.2, 0.4, 0.6, 0.8}, beta in {0.1, ..., 0.5}, gamma in {0, 0.25, 0.5, 0.75} ([paper] §4.2), as
    float64 values of the decimal literals."""
    alphas = (0.2, 0.4, 0.6, 0.8)
    betas = (0.1, 0.2, 0.3, 0.4, 0.5)
    gammas = (0.0, 0.25, 0.5, 0.75)
    vals = [(a, b, g) for a in alphas for b in betas for g in gammas]
    return torch.tensor(vals, dtype=torch.float64, device=device)


def calibrate(scores: torch.Tensor, topk: int, grid: Optional[torch.Tensor] = None, ws: Optional[Workspace] = None,
              stream=None):
    """Grid search of the predictor parameters over a prefill score matrix scores [rows][blocks] (fp32,
    device).  Returns (H [n] fp64 device tensor, best [1] int32 device tensor)."""
    lib = load_library()
    rows, blocks = scores.shape
    if grid is None:
        grid = calibration_grid(scores.device)
    n = grid.shape[0]
    H = torch.empty(n, dtype=torch.float64, device=scores.device)
    best = torch.empty(1, dtype=torch.int32, device=scores.device)
    if ws is None:
        ws = Workspace(lib.prr_calibrate_workspace_bytes(rows, blocks, n), device=scores.device)
    st = lib.prr_calibrate(_ptr(scores), rows, blocks, int(topk), _ptr(grid), n, _ptr(H), _ptr(best), ws.ptr(),
                           ws.nbytes, _stream(stream))
    _check(st, "prr_calibrate")
    return H, best


class BudgetTable:
    """The speculation-budget table ([paper] §4.4, A.6): profiled selection and speculative-attention
    latencies over context lengths `ctx` and budget ratios `deltas` (t_spec[j][i] at deltas[j], ctx[i]),
    with the library's polynomial fit of `degree`.  choose(T) returns (index of the largest delta whose
    speculative latency is at most the selection latency at T tokens, or -1; the estimates).  Host arrays only:
    no GPU work."""

    def __init__(self, ctx, t_select, deltas, t_spec, degree: int = 2):
        import numpy as np

        self.ctx = np.ascontiguousarray(ctx, dtype=np.float64)
        self.t_select = np.ascontiguousarray(t_select, dtype=np.float64)
        self.deltas = np.ascontiguousarray(deltas, dtype=np.float64)
        self.t_spec = np.ascontiguousarray(t_spec, dtype=np.float64)
        if self.t_spec.shape != (len(self.deltas), len(self.ctx)) or self.t_select.shape != self.ctx.shape:
            raise ValueError("t_spec must be [len(deltas)][len(ctx)] and t_select [len(ctx)]")
        self.degree = int(degree)
        self.coef = np.zeros((1 + len(self.deltas), self.degree + 1), dtype=np.float64)
        _check(load_library().prr_budget_fit(*self._table(), self.coef.ctypes.data), "prr_budget_fit")

    def _table(self):
        return (self.ctx.ctypes.data, len(self.ctx), self.t_select.ctypes.data, self.deltas.ctypes.data,
                len(self.deltas), self.t_spec.ctypes.data, self.degree)

    def choose(self, context: float):
        import numpy as np

        est = np.zeros(1 + len(self.deltas), dtype=np.float64)
        choice = ctypes.c_int32(0)
        _check(load_library().prr_budget_choose(*self._table(), self.coef.ctypes.data, float(context),
                                                ctypes.addressof(choice), est.ctypes.data, 0, None),
               "prr_budget_choose")
        return int(choice.value), est

    def budget_blocks(self, context: float, topk: int) -> int:
        """|P| in blocks at `context` tokens for a top-K of `topk` blocks (prr_budget_choose): floor(delta K)
        at the chosen delta, or at the smallest profiled delta when none fits."""
        choice = ctypes.c_int32(0)
        blocks = ctypes.c_int32(0)
        _check(load_library().prr_budget_choose(*self._table(), self.coef.ctypes.data, float(context),
                                                ctypes.addressof(choice), None, int(topk), ctypes.addressof(blocks)),
               "prr_budget_choose")
        return int(blocks.value)
