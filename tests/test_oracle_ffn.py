"""Pins of the oracle's expert FFN and of the whole layer."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import numerics as nx


def test_silu_closed_form():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(oracle.silu(-2.0) - (-2.0) * 0.11920292202211755) < 1e-16
    assert oracle.silu(-800.0) == 0.0 and oracle.silu(800.0) == 800.0


def test_expert_ffn_is_dense_swiglu_torch():
    """One expert reduces to a dense SwiGLU FFN: F.linear / F.silu in fp64."""
    rng = np.random.default_rng(0)
    n, H, I = 7, 24, 40                                     # I != H catches transposes
    X, Wg, Wu = rng.normal(size=(n, H)), rng.normal(size=(I, H)), rng.normal(size=(I, H))
    Wd = rng.normal(size=(H, I))
    y = oracle.expert_ffn(X, Wg, Wu, Wd, "f32", "f32")
    tX, tg, tu, td = (torch.from_numpy(a) for a in (X, Wg, Wu, Wd))
    h = (F.silu(F.linear(tX, tg)) * F.linear(tX, tu)).float().double()
    ref = F.linear(h, td).float().double().numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)


def test_expert_ffn_brute_force_loops():
    rng = np.random.default_rng(1)
    n, H, I = 3, 5, 4
    X, Wg, Wu, Wd = (rng.normal(size=s) for s in ((n, H), (I, H), (I, H), (H, I)))
    y = oracle.expert_ffn(X, Wg, Wu, Wd, "f32", "f32")
    for r in range(n):
        h = []
        for i in range(I):
            g = sum(X[r][j] * Wg[i][j] for j in range(H))
            u = sum(X[r][j] * Wu[i][j] for j in range(H))
            h.append(float(np.float32(g / (1 + math.exp(-g)) * u)))
        for j in range(H):
            assert abs(y[r][j] - sum(h[i] * Wd[j][i] for i in range(I))) < 1e-5


def test_bf16_roundings_at_stated_points():
    rng = np.random.default_rng(2)
    n, H, I = 6, 32, 16
    X = nx.to_bf16(rng.normal(size=(n, H)))
    Wg, Wu = nx.to_bf16(rng.normal(size=(I, H))), nx.to_bf16(rng.normal(size=(I, H)))
    Wd = nx.to_bf16(rng.normal(size=(H, I)))
    y = oracle.expert_ffn(X, Wg, Wu, Wd, "bf16", "bf16")
    h = nx.to_bf16(oracle.silu(X @ Wg.T) * (X @ Wu.T))
    np.testing.assert_array_equal(y, nx.to_bf16(h @ Wd.T))
    np.testing.assert_array_equal(nx.to_bf16(y), y)


def test_single_expert_layer_is_dense_ffn():
    """E = 1, K = 1: every token goes to the one expert with gate 1, and the
    layer is the dense SwiGLU FFN of torch."""
    rng = np.random.default_rng(3)
    T, H, I = 11, 16, 24
    x = rng.normal(size=(T, H))
    W = [rng.normal(size=s) for s in ((I, H), (I, H), (H, I))]
    res = oracle.layer(x, rng.normal(size=(T, 1)).astype(np.float32), 1, 1, 0, 1,
                       lambda e: W, "f32", "f32", "f32")
    assert np.all(res["gates"] == 1.0)
    tx = torch.from_numpy(x)
    h = F.silu(F.linear(tx, torch.from_numpy(W[0]))) * F.linear(tx, torch.from_numpy(W[1]))
    ref = F.linear(h, torch.from_numpy(W[2])).numpy()
    np.testing.assert_allclose(res["out"], ref, rtol=1e-5, atol=1e-5)


def test_layer_equals_per_token_sum_over_experts():
    """The permuted, grouped computation equals the unpermuted definition:
    out[t] = sum_k gate[t,k] * FFN_{ids[t,k]}(x[t])."""
    rng = np.random.default_rng(4)
    T, H, I, E, K = 20, 12, 10, 6, 2
    x = rng.normal(size=(T, H))
    Ws = [[rng.normal(size=s) for s in ((I, H), (I, H), (H, I))] for _ in range(E)]
    lg = rng.normal(size=(T, E)).astype(np.float32)
    res = oracle.layer(x, lg, K, E, 0, E, lambda e: Ws[e], "f32", "f32", "f32")
    for t in range(T):
        acc = np.zeros(H)
        for k in range(K):
            e = res["ids"][t, k]
            acc += np.float32(res["gates"][t, k]) * oracle.expert_ffn(x[t:t + 1], *Ws[e], "f32", "f32")[0]
        np.testing.assert_allclose(res["out"][t], acc, rtol=1e-6, atol=1e-6)


def test_layer_local_range_offsets_expert_index():
    """With local experts [e0, e1), weights_of(j) is local expert j = e0 + j."""
    rng = np.random.default_rng(5)
    T, H, I, E, K, e0, e1 = 30, 8, 8, 8, 2, 4, 8
    x = rng.normal(size=(T, H))
    Ws = [[rng.normal(size=s) for s in ((I, H), (I, H), (H, I))] for _ in range(E)]
    lg = rng.normal(size=(T, E)).astype(np.float32)
    res = oracle.layer(x, lg, K, E, e0, e1, lambda j: Ws[e0 + j], "f32", "f32", "f32")
    for t in range(T):
        acc = np.zeros(H)
        for k in range(K):
            e = res["ids"][t, k]
            if e0 <= e < e1:
                acc += np.float32(res["gates"][t, k]) * oracle.expert_ffn(x[t:t + 1], *Ws[e], "f32", "f32")[0]
        np.testing.assert_allclose(res["out"][t], acc, rtol=1e-6, atol=1e-6)


def test_shared_expert_layer_is_routed_layer_plus_dense_ffn():
    """With one shared expert (every token, gate 1) the layer's output is the
    routed layer's output plus a dense SwiGLU of the shared weights on every
    token -- the latter written with torch's F.linear / F.silu, not the
    oracle's expert code."""
    import torch
    import torch.nn.functional as F
    rng = np.random.default_rng(21)
    T, E, K, H, I = 11, 6, 2, 16, 12
    x = rng.standard_normal((T, H))
    logits = rng.standard_normal((T, E))
    W = [tuple(rng.standard_normal(s) / np.sqrt(s[1]) for s in ((I, H), (I, H), (H, I))) for _ in range(E + 1)]
    routed = oracle.layer(x, logits, K, E, 0, E, lambda e: W[e], "f32", "f32", "f32")
    shared = oracle.layer(x, logits, K, E, 0, E, lambda e: W[e], "f32", "f32", "f32", n_shared=1)
    xt = torch.from_numpy(x)
    g, u, d = (torch.from_numpy(m) for m in W[E])
    dense = F.linear(F.silu(F.linear(xt, g)) * F.linear(xt, u), d).numpy()
    np.testing.assert_allclose(shared["out"], routed["out"] + dense, rtol=1e-5, atol=1e-5)
    ids, gates = oracle.route_shared(logits, K, 1)
    assert (ids[:, K] == E).all() and (gates[:, K] == 1.0).all()
    r_ids, r_g = oracle.route(logits, K)
    np.testing.assert_array_equal(ids[:, :K], r_ids)
    np.testing.assert_array_equal(gates[:, :K], r_g)
