"""Seeded random sweep of whole-layer parity against the oracle.

The named parity cases pin the shapes the workloads and the kernels' tile
families need; this sweep draws further shapes from one seeded generator so
that combinations nobody listed are checked too: activation dtype (fp32,
bf16, fp8 with fp32 or power-of-two weight scales), E from 1 to 300, K from
1 to 70 (capped at E), H and I any multiple of 8 (16 for fp8) up to 1024,
one to three source segments of random length, a random local expert range
in some cases, roughly 2 to 800 rows per local expert (so every tile family
of both GEMM stages and several m-tiles per expert are reached), packed or
dense weights, and in a quarter of the cases the masked layout with a
per-expert capacity that is sometimes smaller than the busiest expert.
Checks are those of the named cases: routing, layout, permutation and
dispatch exact, y and out within the layer tolerance.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from harness import Case, assert_close, gpu_view, run_gpu, to_np
from test_gpu_parity import check_exact_stages

pytestmark = pytest.mark.gpu
C = wl.CONFIGS
SEED = 20261203
N_CASES = 40


def _draw(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        kind = str(rng.choice(["bf16", "bf16", "fp8", "fp8", "f32"]))
        base = {"bf16": C["dsv3_prefill"], "fp8": C["gptoss_fp8"], "f32": C["toy"]}[kind]
        q = 16 if kind == "fp8" else 8
        E = int(rng.choice([1, 2, 4, 8, 16, 32, 64, 128, 256, 300]))
        K = int(min(E, rng.choice([1, 2, 4, 8, 8, 12, 20, 70])))
        H = int(q * rng.integers(1, 1024 // q + 1))
        I = int(q * rng.integers(1, 1024 // q + 1))
        nseg = int(rng.integers(1, 4))
        target = int(rng.choice([2, 10, 40, 100, 200, 300, 400, 800]))   # rows per local expert
        e_b, e_e = 0, E
        if E >= 4 and rng.random() < 0.3:
            e_b = int(rng.integers(0, E // 2))
            e_e = int(rng.integers(e_b + 1, E + 1))
        T = max(1, min(3000, target * (e_e - e_b) // K))
        while T * K > 6000 and T > 1:
            T //= 2
        cuts = np.sort(rng.integers(0, T + 1, size=nseg - 1))
        segs = tuple(int(v) for v in np.diff(np.r_[0, cuts, T]))
        ws = str(rng.choice(["fp32", "pow2"])) if kind == "fp8" else None
        packed = bool(rng.random() < 0.35)
        masked = bool(rng.random() < 0.25)
        cap_e = int(max(1, rng.integers(target // 2, 2 * target + 2))) if masked else None
        name = f"s{c}_{kind}_E{E}_K{K}_H{H}_I{I}_T{T}_loc{e_b}-{e_e}"
        name += (f"_{ws}" if ws else "") + ("_packed" if packed else "") + (f"_masked{cap_e}" if masked else "")
        cfg = wl.scaled(base, name, seg_rows=segs, E=E, K=K, H=H, I=I, e_begin=e_b, e_end=e_e,
                        seed=seed % 100000 + c, w_scales=ws)
        out.append((cfg, packed, cap_e))
    return out


CASES = _draw(N_CASES, SEED)


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


@pytest.mark.parametrize("cfg,packed,cap_e", CASES, ids=[c.name for c, _, _ in CASES])
def test_random_layer_parity(cfg, packed, cap_e):
    import combine_grouped_gemm_amd as m
    print(f"[sweep] {cfg.name} segs={cfg.seg_rows}", flush=True)
    case = Case(cfg)
    if packed:
        for k in ("gate", "up", "down"):
            case.wdict[k] = m.moe_pack_weights(case.wdict[k])
    if cap_e is None:
        layer = run_gpu(case)
        g = gpu_view(layer)
        o = case.oracle_layer()
        check_exact_stages(g, o, cfg.act_dtype)
        assert_close(g["y"], o["y"], cfg.act_dtype, "y")
        assert_close(g["out"], o["out"], cfg.act_dtype, "out")
    else:
        layer = m.MoELayer(cfg.seg_rows, cfg.E, cfg.K, cfg.H, cfg.I, cfg.e_begin, cfg.e_end, cfg.act_dtype,
                           cfg.y_dtype, cfg.out_dtype, layout="masked", cap_per_expert=cap_e)
        layer.forward(case.x_dev, case.logits_dev, case.wdict)
        torch.cuda.synchronize()
        o = _oracle_masked(case, layer.cap_e)
        np.testing.assert_array_equal(layer.topk_ids.cpu().numpy(), o["ids"])
        np.testing.assert_array_equal(layer.counts.cpu().numpy(), o["counts"])
        np.testing.assert_array_equal(layer.offsets[:cfg.E_loc].cpu().numpy(), o["m"])
        np.testing.assert_array_equal(layer.row_of.cpu().numpy(), o["row_of"])
        np.testing.assert_array_equal(layer.src_of.cpu().numpy()[:layer.cap], o["src_of"])
        valid = o["src_of"] >= 0
        vrows = torch.as_tensor(np.nonzero(valid)[0], device=layer.y.device)
        np.testing.assert_array_equal(to_np(layer.xd[vrows]), o["xd"][valid])
        if cfg.act_dtype == "fp8":
            np.testing.assert_array_equal(layer.xd_scales.cpu().numpy()[valid], o["xs"][valid])
        assert_close(to_np(layer.y[vrows]), o["y"][valid], cfg.act_dtype, "y")
        assert_close(to_np(layer.out), o["out"], cfg.act_dtype, "out")
    del case, layer
    gc.collect()
    torch.cuda.empty_cache()
