"""Writes ``oracle_lock.json``: a lock table of oracle outputs on small seeded
workloads.  Calls only the oracle and the seeded input generators.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from ssim_loss_amd.inputs import make_workload  # noqa: E402


def main():
    entries = []
    for name, padding, dloss in [("tiny-64", "valid", 1.0), ("tiny-64", "same", 0.5),
                                 ("small-256", "valid", 1.0)]:
        x, y = make_workload(name)
        loss, gx, gy = oracle.ssim_loss(x, y, padding, dloss=dloss)
        rng = np.random.default_rng(1234)
        samples = []
        for _ in range(8):
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            samples.append([list(idx), float(gx[idx]), float(gy[idx])])
        samples.append([[0, 0, 0, 0], float(gx[0, 0, 0, 0]), float(gy[0, 0, 0, 0])])
        entries.append({
            "workload": name, "padding": padding, "dloss": dloss, "loss": loss,
            "abs_sum_gx": float(np.abs(gx).sum()), "abs_sum_gy": float(np.abs(gy).sum()),
            "samples": samples,
        })
    out = {
        "what": "oracle outputs (fp64) on seeded workloads; a lock against unnoticed "
                "changes to the oracle, not an independent pin",
        "entries": entries,
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_lock.json"),
              "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
