"""GPU parity of the layer with always-on shared experts (Moreh report,
"Overview": a shared expert runs for every token regardless of routing),
run as extra groups of the same grouped FFN launch: routing ids and the
layout exact, outputs within the layer's tolerance of the oracle."""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from harness import assert_close, has_gpu, to_np
from oracle import numerics as nx

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

C = wl.CONFIGS
CASES = [
    (C["toy"], 1),
    (wl.scaled(C["dsv3_decode"], "decode_small", seg_rows=(40,), E=32, K=4, H=512, I=256), 1),
    (wl.scaled(C["dsv3_prefill"], "prefill_small", seg_rows=(600,), E=8, K=2, H=384, I=320), 2),
    (wl.scaled(C["gptoss_fp8"], "fp8_small", seg_rows=(300,), E=8, K=2, H=320, I=192), 1),
]


@pytest.mark.parametrize("cfg,ns", CASES, ids=[f"{c.name}-shared{n}" for c, n in CASES])
def test_layer_with_shared_experts(cfg, ns):
    from combine_grouped_gemm_amd import MoELayer
    print(f"[shared] {cfg.name} T={cfg.T} E={cfg.E}+{ns} K={cfg.K}+{ns}", flush=True)
    x_cpu = wl.gen_x(cfg)
    logits_cpu = wl.gen_logits(cfg, x_cpu)
    W = wl.gen_expert_weights(cfg, device="cuda", experts=list(range(cfg.E + ns)))
    w = W.as_dict()
    layer = MoELayer(cfg.seg_rows, cfg.E, cfg.K, cfg.H, cfg.I, 0, cfg.E, cfg.act_dtype, cfg.y_dtype,
                     cfg.out_dtype, n_shared=ns)
    layer.forward([s.cuda() for s in x_cpu], logits_cpu.cuda(), w)
    torch.cuda.synchronize()

    def weights_of(j):
        d = W.expert(j, "cpu")
        if cfg.w_dtype == "fp8":
            return tuple(nx.dequantize_fp8_blocks(to_np(d[k]), to_np(d[k + "_scale"]))
                         for k in ("gate", "up", "down"))
        return tuple(to_np(d[k]) for k in ("gate", "up", "down"))

    x = np.concatenate([to_np(s) for s in x_cpu])
    o = oracle.layer(x, logits_cpu.numpy(), cfg.K, cfg.E, 0, cfg.E, weights_of, cfg.act_dtype,
                     cfg.y_dtype, cfg.out_dtype, n_shared=ns)
    np.testing.assert_array_equal(layer.topk_ids.cpu().numpy(), o["ids"])
    np.testing.assert_allclose(layer.topk_w.cpu().numpy(), o["gates"], rtol=1e-5, atol=1e-7)
    np.testing.assert_array_equal(layer.offsets.cpu().numpy(), o["offsets"])
    np.testing.assert_array_equal(layer.row_of.cpu().numpy(), o["row_of"])
    R = int(o["offsets"][-1])
    assert_close(to_np(layer.y[:R]), o["y"], cfg.act_dtype, "y")
    assert_close(to_np(layer.out), o["out"], cfg.act_dtype, "out")
    del layer, W
    gc.collect()
    torch.cuda.empty_cache()


MB = [
    wl.scaled(C["dsv3_prefill"], "prefill_small", seg_rows=(600,), E=8, K=2, H=384, I=320),
    wl.scaled(C["ep8_share"], "ep_small", seg_rows=(100, 37, 64), E=16, K=3, H=256, I=128,
              e_begin=4, e_end=10),
]


@pytest.mark.parametrize("cfg", MB, ids=[c.name for c in MB])
def test_two_micro_batches_match_single_batch(cfg):
    """Two micro-batches on two streams give the single-batch layer's output
    bit for bit (Moreh report, compute-communication overlapping), and that
    output matches the oracle's layer."""
    from combine_grouped_gemm_amd import MoELayer
    from combine_grouped_gemm_amd.layer import MicroBatchedLayer
    print(f"[micro-batches] {cfg.name} T={cfg.T}", flush=True)
    x = [s.cuda() for s in wl.gen_x(cfg)]
    logits = wl.gen_logits(cfg).cuda()
    W = wl.gen_expert_weights(cfg, device="cuda")
    w = {"gate": W.gate, "up": W.up, "down": W.down}
    args = (cfg.E, cfg.K, cfg.H, cfg.I, cfg.e_begin, cfg.e_end, cfg.act_dtype, cfg.y_dtype, cfg.out_dtype)
    one = MoELayer(cfg.seg_rows, *args)
    ref = one.forward(x, logits, w).clone()
    two = MicroBatchedLayer(cfg.seg_rows, *args)
    for _ in range(2):
        oa, ob = two.forward(x, logits, w)
        torch.cuda.synchronize()
        assert torch.equal(torch.cat([oa, ob]), ref)
    # and against the oracle: each micro-batch routes and lays out its own tokens
    # exactly as the oracle does for them, and the joined output meets the layer's
    # tolerance against the oracle's whole-batch layer
    x_np = np.concatenate([to_np(s) for s in wl.gen_x(cfg)])
    lg_np = wl.gen_logits(cfg).numpy()

    def weights_of(j):
        d = W.expert(j, "cpu")
        return tuple(to_np(d[k]) for k in ("gate", "up", "down"))

    o = oracle.layer(x_np, lg_np, cfg.K, cfg.E, cfg.e_begin, cfg.e_end, weights_of, cfg.act_dtype,
                     cfg.y_dtype, cfg.out_dtype)
    Ta = two.a.T
    for part, rows in ((two.a, slice(0, Ta)), (two.b, slice(Ta, cfg.T))):
        ids_p, _ = oracle.route(lg_np[rows], cfg.K)
        lay_p = oracle.layout(ids_p, cfg.E, cfg.e_begin, cfg.e_end, part.cap)
        np.testing.assert_array_equal(part.topk_ids.cpu().numpy(), ids_p)
        np.testing.assert_array_equal(part.row_of.cpu().numpy(), lay_p["row_of"])
        np.testing.assert_array_equal(part.offsets.cpu().numpy(), lay_p["offsets"])
    np.testing.assert_array_equal(np.concatenate([two.a.topk_ids.cpu().numpy(),
                                                  two.b.topk_ids.cpu().numpy()]), o["ids"])
    assert_close(to_np(torch.cat([oa, ob])), o["out"], cfg.act_dtype, "out (two micro-batches)")
    del one, two, W
    gc.collect()
    torch.cuda.empty_cache()
