"""The C ABI without a GPU: the library loads, exports every symbol the header declares, sizes its
buffers, and rejects bad arguments before anything is enqueued (no compute calls here)."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_quest_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prr.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(prr_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        pytest.fail("libprr.so is not built; run `python -m block_sparse_attention_quest_amd.build`")
    return bd.load_library()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert declared == sorted(bd.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_strerror(lib):
    for code in range(5):
        assert lib.prr_strerror(code)
    assert lib.prr_strerror(99) == b"unknown status"


def _kv(**kw):
    base = dict(k=1, v=1, page_table=1, seq_len=1, batch=2, num_kv_heads=8, head_dim=128, page_size=16,
                num_pages=4096, max_pages=2048, dtype=bd.PRR_BF16)
    base.update(kw)
    return bd.KvCacheStruct(**base)


def test_sizes(lib):
    kv = _kv()
    assert lib.prr_max_blocks(ctypes.byref(kv), 64) == 2048 * 16 // 64
    assert lib.prr_meta_stride(ctypes.byref(kv), 16) == 2048
    kv2 = _kv(max_pages=13)
    assert lib.prr_max_blocks(ctypes.byref(kv2), 16) == 13
    assert lib.prr_meta_stride(ctypes.byref(kv2), 16) == 16
    assert lib.prr_meta_bytes(ctypes.byref(kv), 16) == 2 * 8 * 128 * 2 * 2048 * 2
    ws = lib.prr_attn_workspace_bytes(8, 32, 8, 128, 64, 64)
    assert ws >= 256 + 64 * 4 * (128 + 2) * 4
    assert lib.prr_attn_workspace_bytes(0, 32, 8, 128, 64, 64) == 0


def _set(cap=64):
    return bd.BlockSetStruct(1, 1, cap)


def _state():
    return bd.AttnStateStruct(1, 1, 1)


def test_attention_argument_errors(lib):
    kv = _kv()
    P = _set()
    st = _state()
    ws_need = lib.prr_attn_workspace_bytes(2, 32, 8, 128, 64, 64)
    call = lambda q=1, hq=32, kv=kv, block=64, P=P, out=st, ws=1, wsb=ws_need: lib.prr_spec_attn(
        q, hq, ctypes.byref(kv) if kv is not None else None, block,
        ctypes.byref(P) if P is not None else None, 0.1, ctypes.byref(out) if out is not None else None,
        ws, wsb, None)
    assert call(q=None) == 1
    assert call(kv=None) == 1
    assert call(P=None) == 1
    assert call(out=None) == 1
    assert call(block=24) == 1                          # not a multiple of the page size
    assert call(hq=36) == 1                             # not a multiple of num_kv_heads
    assert call(hq=8 * 32) == 2                         # group of 32 > 16
    assert call(hq=8 * 3) == 2                          # group not a power of two
    assert call(kv=_kv(head_dim=96)) == 2
    assert call(kv=_kv(page_size=32)) == 2
    assert call(kv=_kv(dtype=7)) == 2
    assert call(ws=None) == 3
    assert call(wsb=ws_need - 1) == 3
    assert call(P=bd.BlockSetStruct(1, 1, 0)) == 1
    assert lib.prr_repair(1, 32, ctypes.byref(kv), 64, ctypes.byref(P), 0.1, None, None, 1, ws_need,
                          None) == 1


def test_select_and_predict_argument_errors(lib):
    kv = _kv()
    A = _set(64)
    P = _set(64)
    M = _set(64)
    sel = lambda topk=64, A=A, P=P, M=M, meta=1, kv=kv, block=64, mode=0, ws=None, wsb=0: lib.prr_select(
        1, 32, ctypes.byref(kv), meta, mode, block, topk, ctypes.byref(P) if P else None, 1, ctypes.byref(A),
        ctypes.byref(M) if M else None, ws, wsb, None)
    assert sel(meta=None) == 1
    assert sel(mode=2) == 1                       # unknown score mode
    assert sel(mode=-1) == 1
    assert sel(topk=65) == 1                      # A cap too small
    assert sel(topk=-1) == 1
    assert sel(M=None) == 1                       # P without M
    assert sel(M=_set(10)) == 1
    # rows above 32768 blocks are ranked in part-parallel stages that need the workspace
    long_kv = _kv(max_pages=65536)
    need_sel = lib.prr_select_workspace_bytes(ctypes.byref(long_kv), 0, 16, 64)
    assert need_sel > 0
    assert sel(kv=long_kv, block=16) == 3
    assert sel(kv=long_kv, block=16, ws=1, wsb=need_sel - 1) == 3
    assert sel(kv=_kv(max_pages=131073), block=16) == 2   # more than 131072 blocks per sequence
    pred = lambda budget=64, nmax=2048, P=P, ws=None, wsb=0, kv=None: lib.prr_predict(
        1, 1, 2, 8, 64, nmax, 0.6, 0.3, 0.5, budget, 1, 1, 1, ctypes.byref(P) if P else None,
        ctypes.byref(kv) if kv else None, ws, wsb, None)
    assert pred(budget=65) == 1
    assert pred(P=None) == 1
    # a page work list for P_next needs the cache it maps through, with the predictor's sequences and a
    # block size that divides into pages
    Pl = bd.BlockSetStruct(1, 1, 64, 1)
    assert pred(P=Pl) == 1                                    # no cache
    assert pred(P=Pl, kv=_kv(batch=3)) == 1                   # other sequences
    assert pred(P=Pl, kv=_kv(num_kv_heads=4)) == 1
    assert pred(P=Pl, kv=_kv(page_size=32)) == 2              # unsupported page size
    assert pred(P=Pl, kv=_kv(k=None)) == 1
    # long rows: parts of 512 blocks, min(budget, 512) candidates each, plus counters
    need = lib.prr_predict_workspace_bytes(2, 8, 8192, 64)
    assert need == 256 + 16 * 16 * 64 * 12 + 16 * 16 * 4
    assert lib.prr_predict_workspace_bytes(2, 8, 2048, 64) == 0   # one workgroup per row: none needed
    # more than 4096 candidate slots (64 parts x 256): groups of 8 parts in between, 8 groups per unit
    units = 1 * 8
    stage1 = 256 + units * 64 * 256 * 12 + units * 64 * 4
    assert lib.prr_predict_workspace_bytes(1, 8, 32768, 256) == \
        (stage1 + 255) // 256 * 256 + units * 8 * 256 * 12 + units * 8 * 4
    # above 341 candidates per part, groups of 4096 slots keep the ranking in range up to a budget of 512
    # (400: 10 parts per group, 7 groups); beyond it, one workgroup per unit and no workspace
    stage1 = 256 + units * 64 * 400 * 12 + units * 64 * 4
    assert lib.prr_predict_workspace_bytes(1, 8, 32768, 400) == \
        (stage1 + 255) // 256 * 256 + units * 7 * 400 * 12 + units * 7 * 4
    assert lib.prr_predict_workspace_bytes(1, 8, 32768, 513) == 0
    assert pred(nmax=8192, ws=1, wsb=need - 1) == 3
    assert pred(nmax=40000) == 3                  # a row above 32768 blocks needs the workspace
    assert pred(nmax=140000) == 2                 # above 131072 blocks
    assert pred(nmax=65536, budget=513, P=_set(600)) == 2   # 128 parts of 512 candidates: no plan
    assert lib.prr_build_meta(ctypes.byref(kv), 64, None, None) == 1
    assert lib.prr_build_meta(ctypes.byref(_kv(max_pages=10)), 64, 1, None) == 1   # 160 tokens % 64
    assert lib.prr_build_mean_meta(ctypes.byref(kv), 64, None, None) == 1
    assert lib.prr_build_mean_meta(ctypes.byref(_kv(max_pages=10)), 64, 1, None) == 1
    assert lib.prr_build_mean_meta(None, 64, 1, None) == 1
    # fp32 [B][Hkv][d][stride]: 2 * 8 * 128 * 2048 * 4
    assert lib.prr_mean_meta_bytes(ctypes.byref(kv), 16) == 2 * 8 * 128 * 2048 * 4


def test_calibrate_argument_errors(lib):
    need = lib.prr_calibrate_workspace_bytes(8192, 512, 80)
    assert need >= 80 * 128 * 2 * 512 * 8
    assert lib.prr_calibrate_workspace_bytes(0, 512, 80) == 0
    call = lambda s=1, rows=8192, blocks=512, k=128, grid=1, n=80, H=1, best=1, ws=1, wsb=need: lib.prr_calibrate(
        s, rows, blocks, k, grid, n, H, best, ws, wsb, None)
    assert call(s=None) == 1
    assert call(grid=None) == 1
    assert call(H=None) == 1
    assert call(best=None) == 1
    assert call(rows=0) == 1
    assert call(k=-1) == 1
    assert call(n=0) == 1
    assert call(blocks=4097) == 2
    # rows of 4096 blocks take four waves: the A-set masks grow with them
    assert lib.prr_calibrate_workspace_bytes(100, 4096, 80) >= 100 * 256 * 4 + 80 * 2 * 2 * 4096 * 8
    assert call(n=5000) == 2
    assert call(ws=None) == 3
    assert call(wsb=need - 1) == 3


def test_select_spec_argument_errors(lib):
    kv = _kv()
    A, P, M = _set(64), _set(64), _set(64)
    st = _state()
    need = lib.prr_attn_workspace_bytes(2, 32, 8, 128, 64, 64)
    call = lambda q=1, meta=1, topk=64, P=P, A=A, M=M, out=st, ws=1, wsb=need, kv=kv, block=64, mode=0: lib.prr_select_spec(
        q, 32, ctypes.byref(kv), meta, mode, block, topk, ctypes.byref(P) if P else None, 1,
        ctypes.byref(A) if A else None, ctypes.byref(M) if M else None, 0.1,
        ctypes.byref(out) if out else None, ws, wsb, None)
    assert call(q=None) == 1
    assert call(meta=None) == 1
    assert call(mode=3) == 1
    assert call(P=None) == 1                      # P and M are required
    assert call(M=None) == 1
    assert call(A=None) == 1
    assert call(out=None) == 1
    assert call(topk=65) == 1                     # A and M caps too small
    assert call(M=_set(10)) == 1
    assert call(topk=-1) == 1
    assert call(ws=None) == 3
    assert call(wsb=need - 1) == 3
    assert call(block=24) == 1
    assert call(kv=_kv(max_pages=65536), block=16, wsb=lib.prr_attn_workspace_bytes(2, 32, 8, 128, 16, 64)) == 3
    assert call(kv=_kv(max_pages=131073), block=16) == 2


def test_append_argument_errors(lib):
    kv = _kv()
    sl = kv.seq_len
    call = lambda kv=kv, block=64, k=1, v=1, meta=1, seq=sl, mode=0: lib.prr_append(
        ctypes.byref(kv) if kv is not None else None, block, k, v, meta, mode, seq, None)
    assert call(kv=None) == 1
    assert call(mode=5) == 1
    assert call(k=None) == 1
    assert call(v=None) == 1
    assert call(meta=None) == 1
    assert call(seq=None) == 1
    assert call(seq=sl + 4) == 1                  # must be the cache's own length array
    assert call(block=24) == 1
    assert call(kv=_kv(head_dim=96)) == 2


def test_select_spec_predict_argument_errors(lib):
    """The carried predictor step is checked like prr_predict, and may share no buffer with the selection
    or speculative pass (every call here is rejected before anything is enqueued)."""
    kv = _kv()
    A = bd.BlockSetStruct(0x1000, 0x1100, 64)
    P = bd.BlockSetStruct(0x1200, 0x1300, 64)
    M = bd.BlockSetStruct(0x1400, 0x1500, 64)
    Pn = bd.BlockSetStruct(0x2000, 0x2100, 64)
    st = _state()
    scores = 0x3000
    need = lib.prr_select_spec_workspace_bytes(ctypes.byref(kv), 32, 64, 64, 64)

    def pred(**kw):
        f = dict(scores=0x4000, seq_len=0x4100, batch=2, num_kv_heads=8, block=64, max_blocks=2048, alpha=0.6,
                 beta=0.3, gamma=0.5, budget=64, level=0x4200, trend=0x4300, live=0x4400, P_next=Pn)
        f.update(kw)
        pn = f.pop("P_next")
        return bd.PredictArgsStruct(**f, P_next=ctypes.pointer(pn) if pn is not None else None, ws=None, ws_bytes=0)

    def call(pa):
        return lib.prr_select_spec_predict(1, 32, ctypes.byref(kv), 1, 0, 64, 64, ctypes.byref(P), scores,
                                           ctypes.byref(A), ctypes.byref(M), 0.1, ctypes.byref(st), 1, need,
                                           ctypes.byref(pa), None)

    assert call(pred(scores=None)) == 1
    assert call(pred(live=None)) == 1
    assert call(pred(P_next=None)) == 1
    assert call(pred(budget=65)) == 1                 # P_next cap too small
    assert call(pred(budget=-1)) == 1
    assert call(pred(batch=0)) == 1
    assert call(pred(max_blocks=40000)) == 3          # a long row's predictor needs its workspace
    assert call(pred(max_blocks=140000)) == 2
    # shared buffers
    assert call(pred(scores=scores)) == 1
    assert call(pred(level=scores)) == 1
    assert call(pred(trend=0x1000)) == 1              # A's indices
    assert call(pred(P_next=bd.BlockSetStruct(0x1200, 0x2100, 64))) == 1   # writes the P being read
    assert call(pred(P_next=bd.BlockSetStruct(0x2000, 0x1500, 64))) == 1   # M's counts
    # the selection's own checks still apply
    assert lib.prr_select_spec_predict(1, 32, ctypes.byref(kv), 1, 0, 64, 64, ctypes.byref(P), scores,
                                       ctypes.byref(A), ctypes.byref(M), 0.1, ctypes.byref(st), 1, need - 1,
                                       ctypes.byref(pred()), None) == 3


def test_select_spec_workspace_for_three_stage_rows(lib):
    """Rows with more candidate slots than one ranking holds (32768 blocks at K = 256: 64 parts of 256
    candidates) need room for the groups' candidates and a group arrival counter per unit on top of the
    parts' candidates; shorter rows (8192 blocks: two stages) do not."""
    long_kv = _kv(max_pages=32768)    # 32768 blocks of 16 tokens
    short_kv = _kv(max_pages=8192)    # 8192 blocks
    attn = lambda kv: lib.prr_attn_workspace_bytes(kv.batch, 32, kv.num_kv_heads, kv.head_dim, 16, 256)
    units = long_kv.batch * long_kv.num_kv_heads
    parts1 = units * 64
    stage1 = parts1 * 256 * 12 + parts1 * 4
    groups = units * 8
    three = (stage1 + 255) // 256 * 256 + (groups * 256 * 12 + groups * 4 + 255) // 256 * 256 \
        + (units * 4 + 255) // 256 * 256 + (groups * 4 + 255) // 256 * 256
    need_long = lib.prr_select_spec_workspace_bytes(ctypes.byref(long_kv), 32, 16, 256, 256)
    assert need_long == attn(long_kv) + (three + 255) // 256 * 256 + 256
    parts2 = units * 16
    two = parts2 * 256 * 12 + parts2 * 4
    need_short = lib.prr_select_spec_workspace_bytes(ctypes.byref(short_kv), 32, 16, 256, 256)
    assert need_short == attn(short_kv) + (two + 255) // 256 * 256 + 256


def _stage_bytes(units, nparts, kl, ng, kl2):
    """The three-stage top-K's memory: part candidates (12 bytes a slot, 4 a count), group candidates,
    one group arrival counter per unit, one part arrival counter per group, each rounded up to 256
    bytes."""
    up = lambda x: (x + 255) // 256 * 256
    return up(units * nparts * (kl * 12 + 4)) + up(units * ng * (kl2 * 12 + 4)) + up(units * 4) + up(units * ng * 4)


def test_select_workspace_for_long_rows(lib):
    """prr_select uses a workspace for rows above 8192 blocks (and needs one above 32768).  Each scoring
    workgroup's part
    (512 blocks with bf16 queries or block means, 256 with fp32 min/max, 1024 for bf16 min/max rows of
    32768 blocks and more) keeps min(K, part) candidates; groups of up to 2048 candidate slots (at most 256
    parts) keep K each; then one ranking of the groups' candidates, which must fit 4096 slots."""
    assert lib.prr_select_workspace_bytes(ctypes.byref(_kv(max_pages=8192)), 0, 16, 64) == 0
    # 16384 blocks: optional (the stages are faster with few units); 32 parts, one group of 2048 slots
    assert lib.prr_select_workspace_bytes(ctypes.byref(_kv(max_pages=16384)), 0, 16, 64) == _stage_bytes(16, 32, 64, 1, 64)
    kv = _kv(max_pages=65536)              # 65536 blocks of 16 tokens, 2 x 8 units
    # bf16: 64 wide parts of 64 candidates, groups of 32 parts -> 2 groups of 64
    assert lib.prr_select_workspace_bytes(ctypes.byref(kv), 0, 16, 64) == _stage_bytes(16, 64, 64, 2, 64)
    # fp32 min/max: 256 parts of 256 blocks
    kv32 = _kv(max_pages=65536, dtype=bd.PRR_F32)
    assert lib.prr_select_workspace_bytes(ctypes.byref(kv32), 0, 16, 64) == _stage_bytes(16, 256, 64, 8, 64)
    # fp32 block means: parts of 512
    assert lib.prr_select_workspace_bytes(ctypes.byref(kv32), 1, 16, 64) == _stage_bytes(16, 128, 64, 4, 64)
    # bf16 block means: parts of 512 too (wide parts are for min/max metadata only)
    assert lib.prr_select_workspace_bytes(ctypes.byref(kv), 1, 16, 64) == _stage_bytes(16, 128, 64, 4, 64)
    # K = 256: groups of 8 parts (2048 slots), 8 groups of 256 -> 2048 slots in the ranking
    assert lib.prr_select_workspace_bytes(ctypes.byref(kv), 0, 16, 256) == _stage_bytes(16, 64, 256, 8, 256)
    # 131072 blocks at K = 256: 128 wide parts, 16 groups of 8 parts -> 4096 slots in the ranking
    kv2m = _kv(max_pages=131072, batch=1, num_kv_heads=2)
    assert lib.prr_select_workspace_bytes(ctypes.byref(kv2m), 0, 16, 256) == _stage_bytes(2, 128, 256, 16, 256)
    # ... with block means (parts of 512): groups of 2048 slots would leave 32 x 256 to rank, so groups
    # of 16 parts
    assert lib.prr_select_workspace_bytes(ctypes.byref(kv2m), 1, 16, 256) == _stage_bytes(2, 256, 256, 16, 256)
    # K = 512 at 65536 blocks: groups of 4 wide parts would leave 16 x 512 to rank, so groups of 8 parts
    # (4096 slots) leave 8 x 512
    assert lib.prr_select_workspace_bytes(ctypes.byref(kv), 0, 16, 512) == _stage_bytes(16, 64, 512, 8, 512)
    # K = 1024 at 65536 blocks: 16 groups of 1024 is more than one ranking holds: no plan, no workspace
    assert lib.prr_select_workspace_bytes(ctypes.byref(kv), 0, 16, 1024) == 0
    A = _set(1024)
    assert lib.prr_select(1, 32, ctypes.byref(kv), 1, 0, 16, 1024, None, 1, ctypes.byref(A), None, 1, 1 << 30,
                          None) == 2

