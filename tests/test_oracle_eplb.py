"""Pins of the oracle's expert placement (Moreh report, load balancing
between GPUs: 256 experts regrouped into 8 sets of 32 with balanced
activation totals; imbalance from up to 2x down to within 5%)."""
import itertools

import numpy as np
import pytest

import oracle
from oracle import eplb
import workloads as wl


def _is_valid(phys, E):
    return sorted(int(p) for p in phys) == list(range(E))


@pytest.mark.parametrize("E,G,seed", [(8, 2, 0), (16, 4, 1), (256, 8, 2), (12, 3, 3), (5, 5, 4), (7, 1, 5)])
def test_placement_is_a_permutation_with_equal_group_sizes(E, G, seed):
    load = np.random.default_rng(seed).integers(0, 1000, size=E)
    phys = eplb.balanced_placement(load, G)
    assert _is_valid(phys, E)
    S = E // G
    sizes = np.bincount(np.asarray(phys) // S, minlength=G)
    assert (sizes == S).all()
    assert eplb.group_loads(load, phys, G).sum() == load.sum()


def test_placement_rejects_uneven_groups():
    with pytest.raises(ValueError):
        eplb.balanced_placement(np.ones(10), 3)


def test_known_perfect_split():
    # 8..1 into two groups of four: {8,5,4,1} and {7,6,3,2} both sum to 18
    load = np.array([8, 7, 6, 5, 4, 3, 2, 1])
    gl = eplb.group_loads(load, eplb.balanced_placement(load, 2), 2)
    assert list(gl) == [18, 18]


def test_hand_worked_placement():
    """The reading's steps by hand, E = 8 into 2 groups of 4,
    load = [18, 4, 1, 19, 25, 29, 11, 27].  Greedy by decreasing load:
    e5(29) -> g0; e7(27) -> g1; e4(25) -> g1 (27 < 29); e3(19) -> g0 (29 < 52);
    e0(18) -> g0 (48 < 52); e6(11) -> g1 (52 < 66); e1(4) -> g1 (63 < 66, now
    full); e2(1) -> g0.  Groups {0, 2, 3, 5} and {1, 4, 6, 7} both hold 67, so
    no swap; physical ids follow ascending logical id inside each group."""
    load = [18, 4, 1, 19, 25, 29, 11, 27]
    phys = eplb.balanced_placement(load, 2)
    assert list(phys) == [0, 4, 1, 2, 5, 3, 6, 7]
    assert list(eplb.group_loads(load, phys, 2)) == [67, 67]


def test_equal_loads_are_perfectly_balanced_and_keep_order():
    load = np.full(32, 7)
    phys = eplb.balanced_placement(load, 4)
    assert eplb.balance_stats(eplb.group_loads(load, phys, 4))["balancedness"] == 1.0
    assert _is_valid(phys, 32)


def _optimal_max(load, G):
    """Exhaustive minimum over equal-cardinality partitions of the largest group load."""
    E = len(load)
    S = E // G
    best = None

    def rec(rest, acc_max):
        nonlocal best
        if not rest:
            best = acc_max if best is None else min(best, acc_max)
            return
        first = rest[0]
        for comb in itertools.combinations(rest[1:], S - 1):
            grp = (first,) + comb
            s = sum(load[i] for i in grp)
            m = max(acc_max, s)
            if best is not None and m >= best:
                continue
            rec([i for i in rest if i not in grp], m)
    rec(list(range(E)), 0)
    return best


@pytest.mark.parametrize("E,G", [(6, 3), (8, 2), (8, 4), (9, 3), (10, 2)])
def test_placement_close_to_exhaustive_optimum(E, G):
    """Brute force over all equal-cardinality partitions of small instances:
    the heuristic's largest group is never more than 10% (or one smallest
    expert load) above the optimum, and matches it in most instances."""
    rng = np.random.default_rng(E * 100 + G)
    hits = 0
    for _ in range(40):
        load = [int(v) for v in rng.integers(1, 100, size=E)]
        opt = _optimal_max(load, G)
        got = int(eplb.group_loads(load, eplb.balanced_placement(load, G), G).max())
        assert got >= opt
        assert got <= max(opt * 1.10, opt + min(load)), (load, got, opt)
        hits += got == opt
    assert hits >= 20


def _counts(logits, K, E):
    ids, _ = oracle.route(logits.numpy(), K)
    return np.bincount(ids.reshape(-1), minlength=E), ids


def test_ep8_share_routing_imbalance_drops_to_within_5_percent():
    """The EP-share workload's routing is calibrated so contiguous 32-expert
    groups differ in load by 2x (the report's "up to 2x", as max/min).
    Placement from the activation counts of 8 calibration batches (same
    model and bias, other tokens) brings 8 other batches within the report's
    5% by the same measure.  (One batch alone still carries ~2% sampling noise
    per group: its balance is reported, not pinned.)"""
    cfg = wl.CONFIGS["ep8_share"]
    E, K, G = cfg.E, cfg.K, 8
    load_c, _ = _counts(wl.gen_calibration_logits(cfg, 1000, batches=8), K, E)
    phys = eplb.balanced_placement(load_c, G)
    load, _ = _counts(wl.gen_calibration_logits(cfg, 2000, batches=8), K, E)
    before = eplb.balance_stats(eplb.group_loads(load, np.arange(E), G))
    after = eplb.balance_stats(eplb.group_loads(load, phys, G))
    assert before["max_over_min"] >= 1.9, before
    assert after["max_over_min"] <= 1.05, after
    load1, ids = _counts(wl.gen_logits(cfg), K, E)
    assert eplb.balance_stats(eplb.group_loads(load1, phys, G))["max_over_min"] < 1.15
    # the remapped routing routes every slot to the physical id of its expert
    np.testing.assert_array_equal(eplb.remap_ids(ids, phys), np.asarray(phys)[ids])


def test_balance_stats_hand_computed():
    """Per-group loads [3, 1, 2] by hand: max/min = 3/1 = 3, mean = 2 so
    max/mean = 3/2 = 1.5, and SGLang's balancedness mean/max = 2/3.  The three
    figures differ from each other, so an exchanged or inverted formula fails."""
    s = eplb.balance_stats([3, 1, 2])
    assert s["max_over_min"] == 3.0
    assert s["max_over_mean"] == 1.5
    assert abs(s["balancedness"] - 2.0 / 3.0) < 1e-15
    # [4, 1, 1]: max/min 4, mean 2 -> max/mean 2, balancedness 1/2
    s = eplb.balance_stats([4, 1, 1])
    assert (s["max_over_min"], s["max_over_mean"], s["balancedness"]) == (4.0, 2.0, 0.5)
    # a group with no load: max/min is unbounded, the other two stay finite
    s = eplb.balance_stats([2, 0])
    assert s["max_over_min"] == float("inf") and s["max_over_mean"] == 2.0 and s["balancedness"] == 0.5


def test_remap_ids_hand_worked():
    """Logical experts 0..3 placed at physical ids [2, 0, 3, 1] (logical 0 sits
    at physical 2, logical 1 at 0, ...).  Tokens routed to logical [[0, 3],
    [1, 2]] go to physical [[2, 1], [0, 3]].  Reading the table the other way
    round (physical -> logical, i.e. its inverse [1, 3, 0, 2]) would give
    [[1, 2], [3, 0]], so the direction of the map is pinned."""
    phys = np.array([2, 0, 3, 1], dtype=np.int32)
    got = eplb.remap_ids(np.array([[0, 3], [1, 2]]), phys)
    assert got.dtype == np.int32
    assert got.tolist() == [[2, 1], [0, 3]]
    assert got.tolist() != np.argsort(phys)[np.array([[0, 3], [1, 2]])].tolist()
