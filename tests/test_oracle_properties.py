"""Property tests of the oracle on random and tie-heavy inputs (hypothesis).

Each property is checked against a definition written independently of the
oracle's code: route against a per-row brute-force ranking of the experts
and the softmax definition; layout against the counting definition of an
expert-contiguous permutation; the fp8 block quantiser against the format's
grid and error bound.  CPU only.
"""
import numpy as np
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp

import oracle
from oracle import numerics

SETTINGS = settings(max_examples=60, deadline=None)


@st.composite
def logits_and_k(draw):
    B = draw(st.integers(1, 12))
    E = draw(st.integers(1, 24))
    K = draw(st.integers(1, E))
    tie_heavy = draw(st.booleans())
    if tie_heavy:       # values from {-1, 0, 1}: many equal logits in a row
        elems = st.sampled_from([-1.0, 0.0, 1.0])
    else:
        elems = st.floats(-30.0, 30.0, allow_nan=False, allow_infinity=False, width=32)
    lg = draw(hnp.arrays(np.float32, (B, E), elements=elems))
    return lg, K


@SETTINGS
@given(logits_and_k())
def test_route_matches_brute_force_ranking(case):
    lg, K = case
    ids, gates = oracle.route(lg, K)
    B, E = lg.shape
    for t in range(B):
        # rank by (logit descending, id ascending) with a plain sort of tuples
        ranked = sorted(range(E), key=lambda e: (-float(lg[t, e]), e))
        assert list(ids[t]) == ranked[:K]
        sel = np.array([float(lg[t, e]) for e in ranked[:K]])
        ref = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        np.testing.assert_allclose(gates[t], ref, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(gates.sum(axis=1), 1.0, rtol=1e-12)
    assert np.all(np.diff(gates, axis=1) <= 1e-15)     # slots in non-increasing gate order


@st.composite
def ids_case(draw):
    B = draw(st.integers(0, 16))
    E = draw(st.integers(1, 12))
    K = draw(st.integers(1, E))
    rows = []
    for _ in range(B):
        rows.append(draw(st.permutations(list(range(E))))[:K])
    ids = np.array(rows, dtype=np.int32).reshape(B, K)
    e_begin = draw(st.integers(0, E - 1))
    e_end = draw(st.integers(e_begin + 1, E))
    extra = draw(st.integers(0, 5))
    return ids, E, e_begin, e_end, extra


@SETTINGS
@given(ids_case())
def test_layout_is_the_expert_contiguous_permutation(case):
    ids, E, e_begin, e_end, extra = case
    B, K = ids.shape
    local_slots = [(t, k) for t in range(B) for k in range(K) if e_begin <= ids[t, k] < e_end]
    R = len(local_slots)
    lay = oracle.layout(ids, E, e_begin, e_end, R + extra)
    # counts: a plain tally over all experts; offsets: running sums over the local range
    tally = [sum(1 for t in range(B) for k in range(K) if ids[t, k] == e) for e in range(E)]
    assert list(lay["counts"]) == tally
    run, offs = 0, [0]
    for e in range(e_begin, e_end):
        run += tally[e]
        offs.append(run)
    assert list(lay["offsets"]) == offs
    # rows: experts in ascending id, inside an expert the slots in (t, k) order
    expected = sorted(local_slots, key=lambda s: (ids[s[0], s[1]], s[0], s[1]))
    for r, (t, k) in enumerate(expected):
        assert lay["row_of"][t, k] == r
        assert lay["src_of"][r] == t * K + k
    assert np.all(lay["src_of"][R:] == -1)
    for t in range(B):
        for k in range(K):
            if not e_begin <= ids[t, k] < e_end:
                assert lay["row_of"][t, k] == -1


@SETTINGS
@given(hnp.arrays(np.float32, st.tuples(st.integers(1, 4), st.integers(1, 300)),
                  elements=st.floats(-1e4, 1e4, allow_nan=False, allow_infinity=False, width=32)))
def test_fp8_block_quantisation_invariants(v):
    codes, scales = numerics.quantize_fp8_blocks(v)
    nb = scales.shape[-1]
    assert nb == -(-v.shape[-1] // 128)
    # scales are powers of two (exact log2) and codes lie on the e4m3 grid within +-448
    m, _ = np.frexp(scales.astype(np.float64))
    assert np.all(m == 0.5)
    assert np.all(np.abs(codes) <= 448.0)
    np.testing.assert_array_equal(numerics.to_e4m3_sat(codes), codes)
    # each block: the largest magnitude uses the top binade (no smaller power of two fits)
    # and the error is at most half a step of the top binade
    deq = numerics.dequantize_fp8_blocks(codes, scales)
    for b in range(nb):
        blk = v[..., b * 128:(b + 1) * 128].astype(np.float64)
        amax = np.abs(blk).max(axis=-1)
        s = scales[..., b].astype(np.float64)
        nz = amax > 0
        assert np.all(amax[nz] <= 448.0 * s[nz])
        assert np.all((amax[nz] > 224.0 * s[nz]) | (s[nz] == 2.0 ** -127))
        err = np.abs(deq[..., b * 128:(b + 1) * 128] - blk).max(axis=-1)
        assert np.all(err <= 16.0 * s + 1e-300)
