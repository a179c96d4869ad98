"""Calibrate the per-expert logit bias of the lumpy EP-share workload.

Test infrastructure: run by hand (``python -m oracle.calibrate_zipf``); it
writes ``workloads/zipf_bias.json``, which the workload generator reads.  It
routes with the oracle only.

The Moreh report ("Load balancing across GPUs") observes up to a 2x load
difference between GPUs when 256 experts are placed as 8 contiguous chunks of
32.  The workload reproduces that: bias_e = beta * ln(pi(e)^-1.1) for a seeded
permutation pi rotated by a multiple of 32 experts, with beta found by
bisection so that the max/min routed-slot count over the 8 contiguous groups
is 2.0.  The first rotation under which group 0 (the local experts 0-31 of the
simulated rank) comes out the most loaded group is kept: that rank is the
straggler that sets the step time.
"""
from __future__ import annotations

import json
import os

import numpy as np

from . import route
import workloads as wl

TARGET = 2.0
GROUPS = 8


def group_loads(logits: np.ndarray, K: int, E: int) -> np.ndarray:
    ids, _ = route(logits, K)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    return counts.reshape(GROUPS, E // GROUPS).sum(axis=1)


def calibrate(name: str):
    cfg = wl.CONFIGS[name]
    x = wl.gen_x(cfg)

    def measure(beta, shift):
        lg = wl.gen_logits(cfg, x, bias_params=(beta, shift)).numpy()
        loads = group_loads(lg, cfg.K, cfg.E)
        return loads.max() / max(loads.min(), 1), loads

    def bisect(shift):
        lo, hi = 0.0, 4.0
        for _ in range(40):
            mid = 0.5 * (lo + hi)
            if measure(mid, shift)[0] < TARGET:
                lo = mid
            else:
                hi = mid
        return hi

    # The raw router logits are not exchangeable across experts for a finite
    # sample, so the rotation changes the loads: bisect beta for each rotation
    # in turn and keep the first one whose group 0 comes out the most loaded.
    group = cfg.E // GROUPS
    for g in range(GROUPS):
        shift = g * group
        beta = bisect(shift)
        r, loads = measure(beta, shift)
        if int(np.argmax(loads)) == 0:
            return {"beta": beta, "shift": shift, "max_over_min": float(r),
                    "group_loads": [int(v) for v in loads]}
    raise RuntimeError("no rotation makes group 0 the most loaded")


def main():
    out = {"note": "written by oracle/calibrate_zipf.py; see its docstring"}
    for name, cfg in wl.CONFIGS.items():
        if cfg.zipf_bias:
            out[name] = calibrate(name)
            print(name, out[name])
    path = os.path.join(os.path.dirname(wl.__file__), "zipf_bias.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=2)
        f.write("\n")


if __name__ == "__main__":
    main()
