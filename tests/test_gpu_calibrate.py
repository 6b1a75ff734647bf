"""GPU parity of the online predictor calibration ([paper] §4.2; [blog] Eqs. (4)-(5)) against the oracle.

Predicted and true top-K sets are exact on both sides, so H(theta) agrees up to float64 rounding of
the hit-rate sums (checked at 1e-9 relative); theta* must equal the oracle's unless the oracle's two
best candidates are within 1e-12 relative (then either is accepted).
"""
import json
import os

import numpy as np
import pytest
import torch

from _gpu import require_gpu
from block_sparse_attention_quest_amd import binding as bd
from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
H_TOL = 1e-9


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    bd.load_library()


def _run(IS: np.ndarray, k: int, grid: np.ndarray):
    s = torch.from_numpy(np.ascontiguousarray(IS, dtype=np.float32)).cuda()
    g = torch.from_numpy(np.ascontiguousarray(grid, dtype=np.float64)).cuda()
    H, best = bd.calibrate(s, k, g)
    torch.cuda.synchronize()
    return H.cpu().numpy(), int(best.cpu().numpy()[0])


def _check(IS, k, grid, what=""):
    H, best = _run(IS, k, grid)
    oH, obest = orc.calibrate(np.asarray(IS, dtype=np.float32).astype(np.float64), k, grid)
    den = np.maximum(np.abs(oH), 1e-300)
    err = np.max(np.abs(H - oH) / den) if oH.size else 0.0
    assert err <= H_TOL or np.max(np.abs(H - oH)) <= 1e-15, f"{what}: max rel err {err}"
    order = np.argsort(-oH, kind="stable")
    if len(oH) > 1 and abs(oH[order[0]] - oH[order[1]]) <= 1e-12 * abs(oH[order[0]]):
        assert best in (order[0], order[1]), what
    else:
        assert best == obest, f"{what}: best {best} vs {obest}"
    return H, best


def test_hand_worked_fixture():
    g = json.load(open(os.path.join(GOLDEN, "calibration_hand.json")))
    H, best = _run(np.array(g["IS"]), g["k"], np.array(g["grid"]))
    for h, (num, den) in zip(H, g["H_num_den"]):
        assert abs(h - num / den) <= 1e-15
    assert best == g["best"]


@pytest.mark.parametrize("rows,blocks,k,seed", [(300, 100, 17, 1), (129, 64, 8, 2), (200, 512, 128, 3),
                                                (70, 1000, 300, 4), (66, 33, 5, 5), (100, 2000, 100, 6),
                                                (130, 4096, 256, 7), (67, 1025, 1024, 8)])
def test_random_lognormal_full_grid(rows, blocks, k, seed):
    w = wl.scaled(wl.C5, seed=seed)
    IS = wl.make_calibration_scores(w, rows=rows, blocks=blocks)
    _check(IS, k, orc.calibration_grid(), f"{rows}x{blocks} k={k}")


@pytest.mark.parametrize("rows,blocks,k", [(90, 70, 20), (60, 3000, 500)])
def test_integer_ties(rows, blocks, k):
    rng = np.random.default_rng(11)
    IS = rng.integers(1, 4, size=(rows, blocks)).astype(np.float32)
    _check(IS, k, orc.calibration_grid(), f"ties {rows}x{blocks}")


def test_prefill_rows_of_4096_blocks():
    """The pages' 64K-token prefill at 16-token blocks: rows of 4096 blocks (the widest supported), a
    full grid against the oracle ([paper] A.5)."""
    w = wl.scaled(wl.C5, seed=9)
    IS = wl.make_calibration_scores(w, rows=160, blocks=4096)
    _check(IS, 256, orc.calibration_grid(), "160x4096 k=256")


def test_degenerate_cases():
    grid = orc.calibration_grid()
    const = np.full((50, 40), 3.0, dtype=np.float32)
    H, best = _check(const, 10, grid, "constant")
    assert np.all(H == 1.0) and best == 0
    rng = np.random.default_rng(12)
    IS = rng.random((40, 30)).astype(np.float32) + 0.5
    H, _ = _check(IS, 0, grid, "k=0")
    assert np.all(H == 0.0)
    H, _ = _check(IS, 30, grid, "k=N")
    assert np.all(H == 1.0)
    H, best = _check(IS[:1], 5, grid, "one row")
    assert np.all(H == 0.0) and best == 0


def test_full_size_prefill_matrix_against_golden():
    """8192 x 512 lognormal prefill matrix, K = 128, all 80 candidates on the GPU against the oracle's
    stored result (tests/golden/calibration_c5_8192x512.json, written by a script that calls only the
    oracle; its tie to the generator and the oracle is checked on the CPU): every H within 1e-9 relative
    and the same theta*."""
    g = json.load(open(os.path.join(GOLDEN, "calibration_c5_8192x512.json")))
    w = wl.C5
    IS = wl.make_calibration_scores(w)
    grid = orc.calibration_grid()
    H, best = _run(IS, w.topk, grid)
    oH = np.array([float.fromhex(x) for x in g["H_hex"]])
    err = np.abs(H - oH) / oH
    assert np.all(err <= H_TOL), (int(np.argmax(err)), float(err.max()))
    order = np.argsort(-oH, kind="stable")
    if abs(oH[order[0]] - oH[order[1]]) <= 1e-12 * oH[order[0]]:
        assert best in (order[0], order[1])
    else:
        assert best == g["best"], (best, g["best"])
