"""Pins of the oracle's layout, dispatch and combine steps."""
import json
import os

import numpy as np
import pytest

import oracle


def _brute_layout(ids, E, e_begin, e_end, cap):
    """Nested loops: experts in order, then tokens, then slots."""
    B, K = ids.shape
    counts = [0] * E
    for t in range(B):
        for k in range(K):
            counts[int(ids[t, k])] += 1
    offsets = [0]
    for e in range(e_begin, e_end):
        offsets.append(offsets[-1] + counts[e])
    row_of = [[-1] * K for _ in range(B)]
    src_of = [-1] * cap
    r = 0
    for e in range(e_begin, e_end):
        for t in range(B):
            for k in range(K):
                if ids[t, k] == e:
                    row_of[t][k] = r
                    src_of[r] = t * K + k
                    r += 1
    return counts, offsets, row_of, src_of


@pytest.mark.parametrize("B,K,E,e_begin,e_end,seed", [
    (1, 1, 1, 0, 1, 0), (5, 2, 16, 0, 16, 1), (9, 3, 7, 2, 5, 2), (33, 8, 32, 0, 4, 3),
    (40, 4, 12, 11, 12, 4), (64, 2, 16, 0, 16, 5)])
def test_layout_matches_brute_force(B, K, E, e_begin, e_end, seed):
    rng = np.random.default_rng(seed)
    lg = rng.integers(-2, 3, size=(B, E)).astype(np.float32)
    ids, _ = oracle.route(lg, K)
    cap = B * K + 3
    lay = oracle.layout(ids, E, e_begin, e_end, cap)
    counts, offsets, row_of, src_of = _brute_layout(ids, E, e_begin, e_end, cap)
    assert lay["counts"].tolist() == counts
    assert lay["offsets"].tolist() == offsets
    assert lay["row_of"].tolist() == row_of
    assert lay["src_of"].tolist() == src_of


def test_layout_invariants_random():
    rng = np.random.default_rng(7)
    for _ in range(20):
        B, E = int(rng.integers(1, 50)), int(rng.integers(1, 40))
        K = int(rng.integers(1, E + 1))
        e0 = int(rng.integers(0, E)); e1 = int(rng.integers(e0 + 1, E + 1))
        ids, _ = oracle.route(rng.normal(size=(B, E)).astype(np.float32), K)
        lay = oracle.layout(ids, E, e0, e1, B * K)
        assert lay["counts"].sum() == B * K                      # sum of counts is B*K
        R = lay["offsets"][-1]
        assert R == lay["counts"][e0:e1].sum()
        assert np.all(np.diff(lay["offsets"]) == lay["counts"][e0:e1])
        src = lay["src_of"][:R]
        assert sorted(src.tolist()) == sorted(                   # bijection onto local slots
            [i for i, e in enumerate(ids.reshape(-1)) if e0 <= e < e1])
        rf = lay["row_of"].reshape(-1)
        assert np.all(rf[src] == np.arange(R))                   # row_of o src_of = id
        assert np.all(lay["src_of"][R:] == -1)
        for e in range(e0, e1):                                  # rows of an expert ascend in (t, k)
            a, b = lay["offsets"][e - e0], lay["offsets"][e - e0 + 1]
            seg = src[a:b]
            assert np.all(np.diff(seg) > 0)
            assert np.all(ids.reshape(-1)[seg] == e)


def test_toy_figure_empty_experts():
    """The anatomy post's toy figure: 8 ranks, one token each, K=2 of 16, and a
    step in which four experts get no token.  Empty experts are zero-length
    groups in the layout."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "router_rows.json")) as f:
        fig = json.load(f)["toy_figure"]
    E, K, T = fig["E"], fig["K"], fig["ranks"] * fig["tokens_per_rank"]
    # a routing that leaves exactly `empty_experts` experts unused
    used = [e for e in range(E) if e not in (2, 7, 11, 14)]
    ids = np.array([[used[(2 * t) % 12], used[(2 * t + 1) % 12]] for t in range(T)], np.int32)
    lay = oracle.layout(ids, E, 0, E, T * K)
    empty = [e for e in range(E) if lay["counts"][e] == 0]
    assert len(empty) == fig["empty_experts"]
    for e in empty:
        assert lay["offsets"][e] == lay["offsets"][e + 1]
    assert lay["offsets"][-1] == T * K


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_identity_expert_round_trip(act):
    """dispatch -> identity expert -> combine returns x * sum of gates (= x)."""
    rng = np.random.default_rng(3)
    T, H, E, K = 40, 24, 10, 3
    x = oracle.numerics.round_act(rng.normal(size=(T, H)), act)
    ids, gates = oracle.route(rng.normal(size=(T, E)).astype(np.float32), K)
    lay = oracle.layout(ids, E, 0, E, T * K)
    R = int(lay["offsets"][-1])
    xd, _ = oracle.dispatch(x, lay["row_of"], R, act)
    out = oracle.combine(xd, lay["row_of"], gates, act)
    np.testing.assert_array_equal(out, oracle.numerics.round_act(x * gates.sum(1, keepdims=True), act))
    np.testing.assert_allclose(out, x, rtol=1e-6 if act == "f32" else 0)


def test_identity_round_trip_partial_local_range():
    """With only experts [e0, e1) local, the round trip returns x times the sum
    of the local gates; tokens with no local slot come back as 0."""
    rng = np.random.default_rng(4)
    T, H, E, K, e0, e1 = 60, 16, 32, 4, 0, 8
    x = rng.normal(size=(T, H))
    ids, gates = oracle.route(rng.normal(size=(T, E)).astype(np.float32), K)
    lay = oracle.layout(ids, E, e0, e1, T * K)
    xd, _ = oracle.dispatch(x, lay["row_of"], int(lay["offsets"][-1]), "f32")
    out = oracle.combine(xd, lay["row_of"], gates, "f32")
    local = (ids >= e0) & (ids < e1)
    scale = (gates * local).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(out, oracle.numerics.to_f32(x * scale), rtol=1e-7, atol=0)
    assert np.any(~local.any(axis=1))                     # the case occurs
    assert np.all(out[~local.any(axis=1)] == 0)


def test_fp8_dispatch_copies_identical_codes():
    rng = np.random.default_rng(5)
    T, H, E, K = 12, 200, 6, 3
    x = oracle.numerics.to_bf16(rng.normal(size=(T, H)))
    ids, _ = oracle.route(rng.normal(size=(T, E)).astype(np.float32), K)
    lay = oracle.layout(ids, E, 0, E, T * K)
    xd, xs = oracle.dispatch(x, lay["row_of"], T * K, "fp8")
    assert xs.shape == (T * K, 2)
    for t in range(T):
        rows = lay["row_of"][t]
        for r in rows[1:]:
            np.testing.assert_array_equal(xd[r], xd[rows[0]])
            np.testing.assert_array_equal(xs[r], xs[rows[0]])
        deq = oracle.numerics.dequantize_fp8_blocks(xd[rows[0]], xs[rows[0]])
        # e4m3 keeps 3 fraction bits: error <= half a step of the top binade,
        # 16 * s, with the power-of-two scale s < 2 * amax / 448
        amax = np.maximum(np.abs(x[t, :128]).max(), 1e-30)
        assert np.max(np.abs(deq[:128] - x[t, :128])) <= amax / 448 * 32 * 1.0001


# ---------------------------------------------------------------------------
# masked (fixed-capacity) layout
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,K,E,e_begin,e_end,seed", [
    (1, 1, 1, 0, 1, 0), (9, 3, 7, 2, 5, 2), (33, 8, 32, 0, 4, 3), (64, 2, 16, 0, 16, 5),
    (128, 8, 256, 0, 256, 6)])
def test_masked_layout_is_contiguous_layout_in_fixed_blocks(B, K, E, e_begin, e_end, seed):
    """With room for every row, the masked layout is the contiguous one with
    expert j's rows moved from offsets[j] to j*cap_e (the contiguous oracle
    builds its permutation by a stable sort, the masked one by running ranks)."""
    rng = np.random.default_rng(seed)
    ids, _ = oracle.route(rng.standard_normal((B, E)).astype(np.float32), K)
    lay = oracle.layout(ids, E, e_begin, e_end, B * K)
    cap_e = int(max(lay["counts"].max(), 1))
    mk = oracle.layout_masked(ids, E, e_begin, e_end, cap_e)
    np.testing.assert_array_equal(mk["counts"], lay["counts"])
    np.testing.assert_array_equal(mk["m"], np.diff(lay["offsets"]))
    off = lay["offsets"]
    for t in range(B):
        for k in range(K):
            r = lay["row_of"][t, k]
            if r < 0:
                assert mk["row_of"][t, k] == -1
                continue
            j = int(np.searchsorted(off, r, side="right") - 1)
            assert mk["row_of"][t, k] == j * cap_e + (r - off[j])
    # src_of inverts row_of on the valid rows; the rest are -1
    valid = mk["src_of"] >= 0
    assert valid.sum() == off[-1]
    rows = np.nonzero(valid)[0]
    flat = mk["row_of"].reshape(-1)
    np.testing.assert_array_equal(flat[mk["src_of"][rows]], rows)


def test_masked_layout_overflow_keeps_first_slots():
    """An expert with more slots than cap_e keeps its first cap_e slots in
    (t, k) order; the rest are dropped (row_of = -1) but still counted."""
    ids = np.array([[0, 1], [0, 2], [1, 0], [0, 3], [2, 0]], dtype=np.int32)
    mk = oracle.layout_masked(ids, 4, 0, 4, 2)
    np.testing.assert_array_equal(mk["counts"], [5, 2, 2, 1])
    np.testing.assert_array_equal(mk["m"], [2, 2, 2, 1])
    # expert 0 slots in order: (0,0) (1,0) (2,1) (3,0) (4,1) -> first two kept
    assert mk["row_of"][0, 0] == 0 and mk["row_of"][1, 0] == 1
    assert mk["row_of"][2, 1] == -1 and mk["row_of"][3, 0] == -1 and mk["row_of"][4, 1] == -1
    assert mk["row_of"][0, 1] == 2 and mk["row_of"][2, 0] == 3      # expert 1 block starts at 2
    assert mk["row_of"][1, 1] == 4 and mk["row_of"][4, 0] == 5      # expert 2
    assert mk["row_of"][3, 1] == 6                                   # expert 3
    np.testing.assert_array_equal(mk["src_of"], [0, 2, 1, 4, 3, 8, 7, -1])


def test_masked_grouped_ffn_matches_contiguous():
    """The masked grouped FFN on the masked buffer equals the contiguous one
    on the contiguous buffer, row for row."""
    rng = np.random.default_rng(11)
    B, K, E, H, I = 12, 2, 4, 8, 6
    ids, _ = oracle.route(rng.standard_normal((B, E)).astype(np.float32), K)
    x = rng.standard_normal((B, H))
    W = [tuple(rng.standard_normal(s) for s in ((I, H), (I, H), (H, I))) for _ in range(E)]
    lay = oracle.layout(ids, E, 0, E, B * K)
    cap_e = int(lay["counts"].max()) + 1
    mk = oracle.layout_masked(ids, E, 0, E, cap_e)
    xd_c, _ = oracle.dispatch(x, lay["row_of"], B * K, "f32")
    xd_m, _ = oracle.dispatch(x, mk["row_of"], E * cap_e, "f32")
    y_c = oracle.grouped_ffn(xd_c, lay["offsets"], lambda e: W[e], "f32", "f32")
    y_m = oracle.grouped_ffn_masked(xd_m, mk["m"], cap_e, lambda e: W[e], "f32", "f32")
    flat_c, flat_m = lay["row_of"].reshape(-1), mk["row_of"].reshape(-1)
    for s in range(B * K):
        np.testing.assert_array_equal(y_m[flat_m[s]], y_c[flat_c[s]])
