"""Plain CPU oracle of expert placement for load balancing across EP ranks.

Test infrastructure only (see the package header).

Moreh report ("21K output tokens/s DeepSeek inference on AMD Instinct
MI300X GPUs with Expert Parallelism"), section on load balancing between
GPUs: splitting the 256 experts into 8 contiguous chunks (0-31 on the first
GPU, ...) left up to a 2x workload imbalance between GPUs; measuring each
expert's activation frequency and grouping the experts into 8 sets of 32
with totals as equal as possible (a variant of balanced number
partitioning), then renumbering the experts so each set is contiguous and
having the gating network emit the renumbered ids, brought the imbalance
within 5%.  SGLang "Expert Parallelism", workload-balancer section: the
figure of merit is balancedness, mean over max of the per-GPU load.

The pages do not give the grouping algorithm.  The reading used here (the
plainest one that meets the equal-cardinality constraint):

1. greedy: experts in order of decreasing load (ties: lower id first), each
   to the least-loaded group that still has room (ties: lower group index);
2. local search: while the most and the least loaded groups (ties: lower
   index) differ, swap the pair (a from the most loaded, b from the least
   loaded) with 0 < load[a] - load[b] < difference whose load difference is
   closest to half the group difference (ties: lower a, then lower b); stop
   when no such pair exists.  Every swap lowers the sum of squared group
   loads, so the loop ends;
3. renumbering: group g takes the physical ids [g*S, (g+1)*S), S = E/G, its
   experts in ascending logical id.
"""
from __future__ import annotations

import numpy as np


def balanced_placement(load, n_groups: int):
    """phys_of_logical (E,) int32: the physical id of every logical expert."""
    load = [int(v) for v in np.asarray(load).reshape(-1)]
    E = len(load)
    if n_groups < 1 or E % n_groups:
        raise ValueError("E must be a positive multiple of n_groups")
    S = E // n_groups
    # 1. greedy
    groups = [[] for _ in range(n_groups)]
    gl = [0] * n_groups
    for e in sorted(range(E), key=lambda i: (-load[i], i)):
        g = min((g for g in range(n_groups) if len(groups[g]) < S), key=lambda g: (gl[g], g))
        groups[g].append(e)
        gl[g] += load[e]
    # 2. local search between the extreme groups
    while True:
        gmax = max(range(n_groups), key=lambda g: (gl[g], -g))
        gmin = min(range(n_groups), key=lambda g: (gl[g], g))
        diff = gl[gmax] - gl[gmin]
        if diff <= 0:
            break
        best = None
        for a in sorted(groups[gmax]):
            for b in sorted(groups[gmin]):
                d = load[a] - load[b]
                if 0 < d < diff:
                    score = abs(diff - 2 * d)
                    if best is None or score < best[0]:
                        best = (score, a, b, d)
        if best is None:
            break
        _, a, b, d = best
        groups[gmax][groups[gmax].index(a)] = b
        groups[gmin][groups[gmin].index(b)] = a
        gl[gmax] -= d
        gl[gmin] += d
    # 3. renumbering
    phys = np.empty(E, dtype=np.int32)
    for g in range(n_groups):
        for i, e in enumerate(sorted(groups[g])):
            phys[e] = g * S + i
    return phys


def group_loads(load, phys_of_logical, n_groups: int):
    """Total load of each physical group [g*S, (g+1)*S)."""
    load = np.asarray(load, dtype=np.int64).reshape(-1)
    S = len(load) // n_groups
    out = np.zeros(n_groups, dtype=np.int64)
    for e, p in enumerate(np.asarray(phys_of_logical)):
        out[int(p) // S] += load[e]
    return out


def balance_stats(group_load):
    """max/min, max/mean and balancedness (mean/max) of per-group loads."""
    gl = np.asarray(group_load, dtype=np.float64)
    mean, mx, mn = gl.mean(), gl.max(), gl.min()
    return {"max_over_min": float(mx / mn) if mn > 0 else float("inf"),
            "max_over_mean": float(mx / mean) if mean > 0 else 1.0,
            "balancedness": float(mean / mx) if mx > 0 else 1.0}


def remap_ids(ids, phys_of_logical):
    """The routing result in physical ids: phys_of_logical[ids]."""
    return np.asarray(phys_of_logical)[np.asarray(ids)].astype(np.int32)
