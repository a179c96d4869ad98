"""GPU parity of routing through an expert placement map and of the layer
run on a balanced placement (Moreh report, load balancing between GPUs).

Mapped routing must equal the oracle's ids sent through the map, bit for
bit, with unchanged gates; the layer on a placement must match the oracle
run on the remapped ids with each physical slot holding its logical
expert's weights (integers exact, floats within the bf16 tolerance).
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from oracle import eplb
import workloads as wl
from harness import assert_close, has_gpu, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


@pytest.mark.parametrize("B,E,K,seed", [(333, 256, 8, 1), (64, 16, 2, 2), (5, 1024, 8, 3), (0, 32, 4, 4)])
def test_route_mapped_matches_oracle(B, E, K, seed):
    import combine_grouped_gemm_amd as m
    print(f"[route_mapped] B={B} E={E} K={K}", flush=True)
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((B, E)).astype(np.float32)
    lg[:, ::7] = 0.25                                     # plenty of ties
    perm = rng.permutation(E).astype(np.int32)
    logits = torch.from_numpy(lg).cuda()
    ids, w = m.moe_route_mapped(logits, K, torch.from_numpy(perm).cuda())
    ids0, w0 = m.moe_route(logits, K)
    torch.cuda.synchronize()
    o_ids, o_w = oracle.route(lg, K)
    np.testing.assert_array_equal(ids.cpu().numpy(), eplb.remap_ids(o_ids, perm))
    assert torch.equal(w, w0)
    np.testing.assert_allclose(w.cpu().numpy(), o_w, rtol=1e-5, atol=1e-7)
    np.testing.assert_array_equal(ids0.cpu().numpy(), o_ids)


def test_layer_on_balanced_placement():
    from combine_grouped_gemm_amd import MoELayer, moe_eplb_place
    cfg = wl.scaled(wl.CONFIGS["ep8_share"], "ep_placement_small", seg_rows=(200, 150, 90), E=32, K=4,
                    H=256, I=128, e_begin=0, e_end=8)
    print(f"[placement] {cfg.name} T={cfg.T} E={cfg.E} K={cfg.K} local {cfg.e_begin}..{cfg.e_end}", flush=True)
    x_cpu = wl.gen_x(cfg)
    logits_cpu = wl.gen_logits(cfg, x_cpu)
    # placement from the activation counts of another batch of the same model
    ids_c, _ = oracle.route(wl.gen_calibration_logits(cfg).numpy(), cfg.K)
    phys = moe_eplb_place(np.bincount(ids_c.reshape(-1), minlength=cfg.E), 4).numpy()
    logical_of_phys = np.argsort(phys)
    local_logical = [int(e) for e in logical_of_phys[cfg.e_begin:cfg.e_end]]
    W = wl.gen_expert_weights(cfg, device="cuda", experts=local_logical)
    w = W.as_dict()
    layer = MoELayer(cfg.seg_rows, cfg.E, cfg.K, cfg.H, cfg.I, cfg.e_begin, cfg.e_end, cfg.act_dtype,
                     cfg.y_dtype, cfg.out_dtype)
    layer.expert_map = torch.from_numpy(phys.astype(np.int32)).cuda()
    layer.forward([s.cuda() for s in x_cpu], logits_cpu.cuda(), w)
    torch.cuda.synchronize()
    # oracle: route on logical ids, renumber, then the layer on the physical range
    ids, gates = oracle.route(logits_cpu.numpy(), cfg.K)
    pids = eplb.remap_ids(ids, phys)
    lay = oracle.layout(pids, cfg.E, cfg.e_begin, cfg.e_end, cfg.cap)
    x = np.concatenate([to_np(s) for s in x_cpu])
    R = int(lay["offsets"][-1])
    xd, _ = oracle.dispatch(x, lay["row_of"], R, cfg.act_dtype)

    def weights_of(j):
        d = W.expert(j, "cpu")
        return tuple(to_np(d[k]) for k in ("gate", "up", "down"))

    y = oracle.grouped_ffn(xd, lay["offsets"], weights_of, cfg.act_dtype, cfg.y_dtype)
    out = oracle.combine(y, lay["row_of"], oracle.numerics.round_act(gates, "f32"), cfg.out_dtype)
    np.testing.assert_array_equal(layer.topk_ids.cpu().numpy(), pids)
    np.testing.assert_array_equal(layer.counts.cpu().numpy(), lay["counts"])
    np.testing.assert_array_equal(layer.offsets.cpu().numpy(), lay["offsets"])
    np.testing.assert_array_equal(layer.row_of.cpu().numpy(), lay["row_of"])
    assert_close(to_np(layer.y[:R]), y, cfg.act_dtype, "y")
    assert_close(to_np(layer.out), out, cfg.act_dtype, "out")
    del layer, W
    gc.collect()
    torch.cuda.empty_cache()
