"""Planted mistakes in the oracle (on the CPU) must trip its pins.

Each case swaps one oracle function for a plausibly wrong variant and checks
that at least one of the pin tests then fails."""
import numpy as np
import pytest

import oracle
import oracle.moe as om
from oracle import numerics as nx

import test_oracle_route as tr
import test_oracle_layout as tl
import test_oracle_ffn as tf


def _route_ties_high(logits, K):
    lg = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-lg[:, ::-1], axis=1, kind="stable")
    order = lg.shape[1] - 1 - order                      # ties -> higher id first
    ids = order[:, :K].astype(np.int32)
    sel = np.take_along_axis(lg, order[:, :K], axis=1)
    ex = np.exp(sel - sel[:, :1])
    return ids, ex / ex.sum(axis=1, keepdims=True)


def _route_full_softmax_gates(logits, K):
    ids, _ = _ORIG_ROUTE(logits, K)
    lg = np.asarray(logits, dtype=np.float64)
    full = np.exp(lg - lg.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    return ids, np.take_along_axis(full, ids, axis=1)   # forgot to renormalise


def _layout_unstable(ids, E, e_begin, e_end, cap):
    res = _ORIG_LAYOUT(ids, E, e_begin, e_end, cap)
    src = res["src_of"].copy()
    off = res["offsets"]
    for e in range(len(off) - 1):                        # reverse rows inside each expert
        src[off[e]:off[e + 1]] = src[off[e]:off[e + 1]][::-1]
    row_of = np.full(ids.size, -1, np.int32)
    R = off[-1]
    row_of[src[:R]] = np.arange(R)
    res["src_of"], res["row_of"] = src, row_of.reshape(ids.shape)
    return res


def _silu_sign(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(z))


def _expert_ffn_gate_up_swapped(X, Wg, Wu, Wd, h_dtype, y_dtype):
    return _ORIG_FFN(X, Wu, Wg, Wd, h_dtype, y_dtype)


def _combine_no_gates(y, row_of, gates, out_dtype):
    return _ORIG_COMBINE(y, row_of, np.ones_like(np.asarray(gates, dtype=np.float64)), out_dtype)


_ORIG_ROUTE, _ORIG_LAYOUT, _ORIG_FFN, _ORIG_COMBINE = om.route, om.layout, om.expert_ffn, om.combine


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


@pytest.mark.parametrize("target,bad,pins", [
    ("route", _route_ties_high, [(tr.test_topk_exhaustive_ties, 3), (tr.test_random_rows_match_brute_force,)]),
    ("route", _route_full_softmax_gates, [(tr.test_worked_rows_closed_form_gates,)]),
    ("layout", _layout_unstable, [(tl.test_layout_matches_brute_force, 33, 8, 32, 0, 4, 3)]),
    ("silu", _silu_sign, [(tf.test_silu_closed_form,), (tf.test_expert_ffn_is_dense_swiglu_torch,)]),
    ("expert_ffn", _expert_ffn_gate_up_swapped, [(tf.test_single_expert_layer_is_dense_ffn,)]),
    ("combine", _combine_no_gates, [(tl.test_identity_round_trip_partial_local_range,)]),
])
def test_planted_mistake_is_caught(monkeypatch, target, bad, pins):
    monkeypatch.setattr(om, target, bad)
    monkeypatch.setattr(oracle, target, bad)
    assert any(_fails(p[0], *p[1:]) for p in pins)
