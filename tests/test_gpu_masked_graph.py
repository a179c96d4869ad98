"""GPU parity of the fixed-capacity (masked) layout path, and HIP-graph
replay of the whole layer, through the C ABI.

Masked layout: counts, m, row_of and src_of must equal the oracle's
bit for bit; dispatched rows are bit-exact copies (fp8: identical codes and
scales); y on the valid rows and out meet the layer's tolerance.

Graph replay: the six calls of one layer step captured once and replayed;
every replay (after clearing the outputs, with eager steps and host
synchronisations in between) must reproduce the eager result bit for bit,
since every kernel is deterministic, and each replay's output is also
checked against the oracle's layer (row_of exact, out within tolerance).
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from harness import Case, assert_close, has_gpu, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

C = wl.CONFIGS
MASKED = [
    (C["toy"], None),
    (wl.scaled(C["dsv3_decode"], "decode_small", seg_rows=(40,), E=32, K=4, H=512, I=256), None),
    (wl.scaled(C["dsv3_decode"], "decode_masked_overflow", seg_rows=(96,), E=8, K=2, H=256, I=128), 20),
    (wl.scaled(C["ep8_share"], "ep_small", seg_rows=(100, 37, 64), E=16, K=3, H=256, I=128,
               e_begin=4, e_end=10), 64),
    (wl.scaled(C["dsv3_prefill"], "prefill_small_masked", seg_rows=(600,), E=8, K=2, H=384, I=320), 200),
    (wl.scaled(C["gptoss_fp8"], "fp8_small", seg_rows=(300,), E=8, K=2, H=320, I=192), None),
    # 4096 slots (the single-workgroup layout, four chunks, some blocks overflowing) and
    # 4104 slots (the three-kernel layout), partial expert range
    (wl.scaled(C["ep8_share"], "masked_4096_slots", seg_rows=(300, 212), E=32, K=8, H=128, I=64,
               e_begin=8, e_end=24), 128),
    (wl.scaled(C["ep8_share"], "masked_4104_slots", seg_rows=(300, 213), E=32, K=8, H=128, I=64,
               e_begin=8, e_end=24), 128),
]


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _layer(cfg, **kw):
    from combine_grouped_gemm_amd import MoELayer
    return MoELayer(cfg.seg_rows, cfg.E, cfg.K, cfg.H, cfg.I, cfg.e_begin, cfg.e_end, cfg.act_dtype,
                    cfg.y_dtype, cfg.out_dtype, **kw)


def _oracle_masked(case, cap_e):
    c = case.cfg
    ids, gates = oracle.route(case.logits_np(), c.K)
    gates_s = oracle.numerics.round_act(gates, "f32")
    mk = oracle.layout_masked(ids, c.E, c.e_begin, c.e_end, cap_e)
    xd, xs = oracle.dispatch(case.x_np(), mk["row_of"], c.E_loc * cap_e, c.act_dtype)
    xv = oracle.numerics.dequantize_fp8_blocks(xd, xs) if c.act_dtype == "fp8" else xd
    y = oracle.grouped_ffn_masked(xv, mk["m"], cap_e, case.oracle_weights, c.act_dtype, c.y_dtype)
    out = oracle.combine(y, mk["row_of"], gates_s, c.out_dtype)
    return dict(ids=ids, xd=xd, xs=xs, y=y, out=out, **mk)


@pytest.mark.parametrize("cfg,cap_e", MASKED, ids=[c.name for c, _ in MASKED])
def test_masked_layer_parity(cfg, cap_e):
    print(f"[masked] {cfg.name} T={cfg.T} E={cfg.E} K={cfg.K} cap_e={cap_e}", flush=True)
    case = Case(cfg)
    layer = _layer(cfg, layout="masked", cap_per_expert=cap_e)
    layer.forward(case.x_dev, case.logits_dev, case.wdict)
    torch.cuda.synchronize()
    o = _oracle_masked(case, layer.cap_e)
    np.testing.assert_array_equal(layer.topk_ids.cpu().numpy(), o["ids"])
    np.testing.assert_array_equal(layer.counts.cpu().numpy(), o["counts"])
    np.testing.assert_array_equal(layer.offsets[:cfg.E_loc].cpu().numpy(), o["m"])
    np.testing.assert_array_equal(layer.row_of.cpu().numpy(), o["row_of"])
    np.testing.assert_array_equal(layer.src_of.cpu().numpy()[:layer.cap], o["src_of"])
    valid = o["src_of"] >= 0
    assert valid.sum() == o["m"].sum()
    # rows of a block past its valid count are never written: convert only the valid ones
    vrows = torch.as_tensor(np.nonzero(valid)[0], device=layer.y.device)
    np.testing.assert_array_equal(to_np(layer.xd[vrows]), o["xd"][valid])
    if cfg.act_dtype == "fp8":
        np.testing.assert_array_equal(layer.xd_scales.cpu().numpy()[valid], o["xs"][valid])
    assert_close(to_np(layer.y[vrows]), o["y"][valid], cfg.act_dtype, "y")
    assert_close(to_np(layer.out), o["out"], cfg.act_dtype, "out")
    del case, layer
    _free()


def test_masked_layout_empty_batch():
    import combine_grouped_gemm_amd as m
    ids = torch.empty((0, 4), dtype=torch.int32, device="cuda")
    r = m.moe_layout_masked(ids, 16, 2, 9, 5)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(r["counts"].cpu().numpy(), np.zeros(16, np.int32))
    np.testing.assert_array_equal(r["m"].cpu().numpy(), np.zeros(7, np.int32))
    np.testing.assert_array_equal(r["src_of"].cpu().numpy(), np.full(35, -1, np.int32))


GRAPH = [
    (wl.scaled(C["dsv3_decode"], "decode_small", seg_rows=(40,), E=32, K=4, H=512, I=256), "contiguous"),
    (wl.scaled(C["dsv3_decode"], "decode_small", seg_rows=(40,), E=32, K=4, H=512, I=256), "masked"),
    (wl.scaled(C["gptoss_fp8"], "fp8_small", seg_rows=(300,), E=8, K=2, H=320, I=192), "contiguous"),
]


@pytest.mark.parametrize("cfg,layout", GRAPH, ids=[f"{c.name}-{l}" for c, l in GRAPH])
def test_graph_replay_matches_eager(cfg, layout):
    print(f"[graph] {cfg.name} layout={layout}", flush=True)
    case = Case(cfg)
    layer = _layer(cfg, layout=layout)
    layer.forward(case.x_dev, case.logits_dev, case.wdict)       # eager; also warms caches
    torch.cuda.synchronize()
    ref_out = layer.out.clone()
    ref_row_of = layer.row_of.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(case.x_dev, case.logits_dev, case.wdict)   # warm-up on the capture stream
        with torch.cuda.graph(g, stream=s):
            layer.forward(case.x_dev, case.logits_dev, case.wdict)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    # the eager result itself against the oracle (layout exact, out within tolerance)
    c = case.cfg
    if layout == "masked":
        o = _oracle_masked(case, layer.cap_e)
    else:
        o = case.oracle_layer()
    np.testing.assert_array_equal(ref_row_of.cpu().numpy(), o["row_of"])
    assert_close(to_np(ref_out), o["out"], c.act_dtype, "out (eager, before capture)")
    for rep in range(3):
        layer.out.zero_()
        layer.row_of.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, ref_out), f"replay {rep}: out differs from the eager result"
        assert torch.equal(layer.row_of, ref_row_of), f"replay {rep}: row_of differs"
        assert_close(to_np(layer.out), o["out"], c.act_dtype, f"out (replay {rep}) against the oracle")
        layer.forward(case.x_dev, case.logits_dev, case.wdict)   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(layer.out, ref_out)
    del g, case, layer
    _free()
