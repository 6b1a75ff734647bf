"""The stored oracle calibration of the 70B-shaped share's prefill matrix (tests/golden/
calibration_c5_8192x512.json, written by tests/golden/make_calibration_golden.py) still describes what
the generator and the oracle produce today ([paper] §4.2; [blog] Eqs. (4)-(5)).

The GPU test of the full 8192 x 512 calibration compares all 80 H values against this file, so it must
stay tied to both sides of its making: the score matrix (by its SHA-256) and the oracle (two candidates,
the stored best and the grid's first, recomputed here and compared bit for bit).
"""
import json
import os
import sys

import numpy as np

from block_sparse_attention_quest_amd import workloads as wl
from oracle import prr_oracle as orc

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))
import make_calibration_golden as mk  # noqa: E402

GOLD = os.path.join(HERE, "golden", "calibration_c5_8192x512.json")


def _load():
    with open(GOLD) as f:
        return json.load(f)


def test_golden_matches_generator_and_grid():
    g = _load()
    IS = wl.make_calibration_scores(wl.C5)
    assert IS.shape == (g["rows"], g["blocks"]) and g["k"] == wl.C5.topk
    assert mk.matrix_sha256(IS) == g["scores_sha256"]
    assert np.array_equal(np.array(g["grid"]), orc.calibration_grid())
    H = np.array([float.fromhex(x) for x in g["H_hex"]])
    assert H.shape == (80,) and np.all((H >= 0.0) & (H <= 1.0))
    assert g["best"] == int(np.argmax(H))


def test_golden_matches_oracle_on_two_candidates():
    g = _load()
    IS = wl.make_calibration_scores(wl.C5).astype(np.float64)
    grid = orc.calibration_grid()
    for j in sorted({0, g["best"]}):
        H, _ = orc.calibrate(IS, g["k"], grid[j:j + 1])
        assert H[0] == float.fromhex(g["H_hex"][j]), j
