"""Write the oracle's calibration result for the 70B-shaped share's prefill matrix (8192 rows x 512 blocks,
K = 128, the 80-point grid) to tests/golden/calibration_c5_8192x512.json.

Only oracle/ computes here ([paper] "Predict, Reuse, and Repair ..." §4.2, prefill trajectory and grid
search; [blog] Eqs. (4)-(5)); the score matrix comes from the seeded input generator, and its SHA-256 is
stored beside the result so that a test can tell when the generator no longer makes the same matrix.
Every H value is stored as a float64 hex string (exact).  About 75 s on one core.

Usage: python tests/golden/make_calibration_golden.py
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from block_sparse_attention_quest_amd import workloads as wl  # noqa: E402
from oracle import prr_oracle as orc  # noqa: E402

OUT = os.path.join(HERE, "calibration_c5_8192x512.json")


def matrix_sha256(IS: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(IS, dtype=np.float32).tobytes()).hexdigest()


def main():
    w = wl.C5
    IS = wl.make_calibration_scores(w)
    grid = orc.calibration_grid()
    t0 = time.time()
    H, best = orc.calibrate(IS.astype(np.float64), w.topk, grid)
    print(f"oracle calibration: {time.time() - t0:.1f} s, best {best}, H* {H[best]:.12f}", flush=True)
    doc = {
        "source": "Predict, Reuse, and Repair (paper text), section 4.2: prefill trajectory, score-weighted hit "
                  "rate and grid search over (alpha, beta, gamma); PRR review blog, Eqs. (4) and (5)",
        "how_derived": "oracle/prr_oracle.py::calibrate on workloads.make_calibration_scores(C5) (8192 x 512 "
                       "fp32 lognormal scores with AR(1) rows), K = 128, the 80-point grid in alpha-major order; "
                       "written by tests/golden/make_calibration_golden.py",
        "rows": int(IS.shape[0]),
        "blocks": int(IS.shape[1]),
        "k": int(w.topk),
        "scores_sha256": matrix_sha256(IS),
        "grid": [[float(x) for x in g] for g in grid],
        "H_hex": [float(h).hex() for h in H],
        "best": int(best),
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
