"""Pins of the oracle's route step against what the pages and mathematics fix."""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "router_rows.json")


def _rows():
    with open(GOLDEN) as f:
        return json.load(f)


def test_worked_rows_route_to_printed_experts():
    """The four worked router rows of the EP-kernel anatomy post (Chinese copy,
    section 'What we need to do', router figure) route to the printed pairs."""
    d = _rows()
    logits = np.array([r["logits"] for r in d["rows"]], dtype=np.float32)
    ids, gates = oracle.route(logits, d["K"])
    for r, got in zip(d["rows"], ids):
        assert sorted(got.tolist()) == sorted(r["assignment"]), r["token"]
    # t0 -> [3, 13], the example spelled out in the text itself
    assert ids[0].tolist() == [3, 13]


def test_worked_rows_closed_form_gates():
    """With two picks a > b the renormalised softmax is (sigmoid(a-b), sigmoid(b-a)).
    t0, t2, t3 have gap 0.4 -> 0.598688 / 0.401312; t1 has gap 0.5 -> 0.622459."""
    d = _rows()
    logits = np.array([r["logits"] for r in d["rows"]], dtype=np.float32)
    _, gates = oracle.route(logits, 2)
    expect = {0: 0.598687660112452, 1: 0.622459331201855, 2: 0.598687660112452,
              3: 0.598687660112452}
    for t, g0 in expect.items():
        # logits are fp32 copies of the printed decimals; the gap differs from
        # the decimal gap by < 1e-7, which moves the gate by < 1e-7
        assert abs(gates[t, 0] - g0) < 1e-6
        assert abs(gates[t, 1] - (1 - g0)) < 1e-6
        a, b = float(logits[t, _rows()["rows"][t]["assignment"][0]]), \
            float(logits[t, _rows()["rows"][t]["assignment"][1]])
        assert abs(gates[t, 0] - 1.0 / (1.0 + math.exp(-(a - b)))) < 1e-15


def _brute_topk(row, K):
    """K rounds of 'take the largest remaining logit, lowest id on ties'."""
    row = [float(v) for v in row]
    taken, out = set(), []
    for _ in range(K):
        best = None
        for e, v in enumerate(row):
            if e in taken:
                continue
            if best is None or v > row[best]:
                best = e
        taken.add(best)
        out.append(best)
    return out


@pytest.mark.parametrize("E", [1, 2, 3, 4, 5])
def test_topk_exhaustive_ties(E):
    """Every logit row in {-1, 0, 1}^E, every K: ids equal the brute force."""
    rows = np.array(list(itertools.product([-1.0, 0.0, 1.0], repeat=E)), dtype=np.float32)
    for K in range(1, E + 1):
        ids, gates = oracle.route(rows, K)
        for r, got in zip(rows, ids):
            assert got.tolist() == _brute_topk(r, K)
        np.testing.assert_allclose(gates.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_negative_zero_ties_with_zero():
    ids, _ = oracle.route(np.array([[-0.0, 0.0, -0.0]], dtype=np.float32), 3)
    assert ids[0].tolist() == [0, 1, 2]


def test_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(0)
    lg = rng.normal(size=(7, 12)).astype(np.float32)
    ids, gates = oracle.route(lg, 12)
    full = softmax(lg.astype(np.float64), axis=1)
    np.testing.assert_allclose(gates, np.take_along_axis(full, ids, axis=1), rtol=1e-13)


def test_gates_are_renormalised_full_softmax():
    rng = np.random.default_rng(1)
    lg = (rng.normal(size=(50, 64)) * 3).astype(np.float32)
    for K in (1, 2, 8):
        ids, gates = oracle.route(lg, K)
        full = softmax(lg.astype(np.float64), axis=1)
        sel = np.take_along_axis(full, ids, axis=1)
        np.testing.assert_allclose(gates, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12)
        # slot order: descending logit
        s = np.take_along_axis(lg, ids, axis=1)
        assert np.all(np.diff(s, axis=1) <= 0)


def test_random_rows_match_brute_force():
    rng = np.random.default_rng(2)
    lg = rng.integers(-3, 4, size=(200, 16)).astype(np.float32)   # many ties
    ids, _ = oracle.route(lg, 4)
    for r, got in zip(lg, ids):
        assert got.tolist() == _brute_topk(r, 4)


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        oracle.route(np.array([[0.0, np.nan]], dtype=np.float32), 1)
