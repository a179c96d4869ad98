"""GPU parity: every stage of the HIP path against the oracle.

Integer outputs (ids, counts, offsets, row_of, src_of) and plain copies
(bf16 / fp32 dispatch) must be bit-exact; fp8 dispatch must reproduce the
oracle's codes and scales exactly (both take the quantisation decision in
fp32); floating outputs must meet the layer's tolerance (bf16: relative L2
<= 1e-2 and max-abs <= 5e-2; fp8: relative L2 <= 3e-2; fp32: 1e-5 / 1e-4).
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from harness import Case, TOL, assert_close, gpu_view, has_gpu, run_gpu, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

C = wl.CONFIGS
SMALL = [
    C["toy"],
    wl.scaled(C["dsv3_decode"], "decode_small", seg_rows=(40,), E=32, K=4, H=512, I=256),
    wl.scaled(C["dsv3_prefill"], "prefill_small", seg_rows=(600,), E=8, K=2, H=384, I=320),
    wl.scaled(C["dsv3_prefill"], "prefill_ntail", seg_rows=(333,), E=6, K=2, H=448, I=192),
    wl.scaled(C["dsv3_prefill"], "prefill_320_row_tiles", seg_rows=(640,), E=4, K=2, H=256, I=192),
    wl.scaled(C["ep8_share"], "ep_small", seg_rows=(100, 37, 64), E=16, K=3, H=256, I=128,
              e_begin=4, e_end=10),
    wl.scaled(C["gptoss_fp8"], "fp8_small", seg_rows=(300,), E=8, K=2, H=320, I=192, w_scales="pow2"),
    wl.scaled(C["gptoss_fp8"], "fp8_small_f32_wscales", seg_rows=(300,), E=8, K=2, H=320, I=192,
              w_scales="fp32"),
    wl.scaled(C["gptoss_fp8"], "fp8_wide_f32_wscales", seg_rows=(600,), E=8, K=2, H=640, I=384,
              w_scales="fp32"),
    wl.scaled(C["gptoss_fp8"], "fp8_decode_real_dims", seg_rows=(24,), E=16, K=4, w_scales="pow2"),
    wl.scaled(C["gptoss_fp8"], "fp8_decode_real_dims_f32_wscales", seg_rows=(24,), E=16, K=4, w_scales="fp32"),
    # H = I = 2880: 23 scale blocks per row (whole-row scale runs) and a 64-wide K tail,
    # 48 rows per expert (the wide fp8 tiles), both weight-scale conventions
    wl.scaled(C["gptoss_fp8"], "fp8_wide_real_dims", seg_rows=(192,), E=8, K=2, w_scales="pow2"),
    wl.scaled(C["gptoss_fp8"], "fp8_wide_real_dims_f32_wscales", seg_rows=(200,), E=8, K=2, w_scales="fp32"),
    # fp8 at DeepSeek dimensions: 56 scale blocks per row (past the wide tiles' scale table),
    # ~32 rows per expert through the 128-row fp8 tiles
    wl.scaled(C["gptoss_fp8"], "fp8_dsv3_dims", seg_rows=(64,), E=16, K=8, H=7168, I=2048),
    # 600 local experts (10..165 rows each) through the wide tiles: more experts than the
    # kernels' 512 threads, so the largest-first expert ranking and the tile prefix take
    # several passes
    wl.scaled(C["dsv3_prefill"], "prefill_many_experts", seg_rows=(4800,), E=600, K=8, H=128, I=64),
    wl.scaled(C["gptoss_fp8"], "fp8_wide_many_experts", seg_rows=(3600,), E=600, K=8, H=256, I=128,
              w_scales="pow2"),
    # H and I not multiples of 64: a partial last k-step (8 of 64 bf16 / f32 elements at
    # H = 200, 8 at I = 136; fp8: 80 of 128 bytes at H = 208, 16 at I = 144) and partial
    # output tiles, through every kernel family: the f32 kernel, the 16- and 128-row
    # register-staged bf16 tiles, the 256- and 320-row bf16 rings and the 16- and 128-row
    # fp8 tiles, both weight-scale conventions (the wide fp8 ring takes K % 128 of 0 or 64
    # only, so the ~100-row fp8 cases here run the 128-row tiles; its 64-byte tail is
    # covered by the H = 320 / I = 192 and H = I = 2880 cases above)
    wl.scaled(C["toy"], "f32_k_tail", seg_rows=(40, 24), E=16, K=2, H=200, I=136),
    wl.scaled(C["dsv3_decode"], "bf16_16row_k_tail", seg_rows=(40,), E=32, K=4, H=200, I=136),
    wl.scaled(C["dsv3_decode"], "bf16_128row_k_tail", seg_rows=(300,), E=16, K=2, H=200, I=136),
    wl.scaled(C["dsv3_prefill"], "bf16_wide256_k_tail", seg_rows=(600,), E=8, K=2, H=200, I=136),
    wl.scaled(C["dsv3_prefill"], "bf16_wide320_k_tail", seg_rows=(640,), E=4, K=2, H=200, I=136),
    wl.scaled(C["gptoss_fp8"], "fp8_16row_k_tail", seg_rows=(24,), E=16, K=2, H=208, I=144, w_scales="pow2"),
    wl.scaled(C["gptoss_fp8"], "fp8_128row_k_tail", seg_rows=(160,), E=16, K=2, H=208, I=144,
              w_scales="fp32"),
    wl.scaled(C["gptoss_fp8"], "fp8_wide_k_tail", seg_rows=(400,), E=8, K=2, H=208, I=144, w_scales="fp32"),
    wl.scaled(C["gptoss_fp8"], "fp8_wide_k_tail_po2", seg_rows=(400,), E=8, K=2, H=208, I=144,
              w_scales="pow2"),
    # more than 8 slots per token: combine gathers in passes of 8 slots (two and three passes)
    wl.scaled(C["dsv3_decode"], "decode_k12", seg_rows=(48,), E=32, K=12, H=256, I=128),
    wl.scaled(C["dsv3_prefill"], "prefill_k20", seg_rows=(40,), E=64, K=20, H=128, I=64),
    # more than 64 slots per token: dispatch and combine read the slot rows 64 at a time
    wl.scaled(C["dsv3_decode"], "decode_k70", seg_rows=(20,), E=128, K=70, H=128, I=64),
    # slots past 64 + 16 and past 64 + 40 with rows of 16 (bf16 H = 128) and 40 (fp8
    # H = 320) vectors: the lanes past the row hold those slots in the second ballot
    wl.scaled(C["dsv3_decode"], "decode_k100_partial_wave", seg_rows=(12,), E=128, K=100, H=128, I=64),
    wl.scaled(C["gptoss_fp8"], "fp8_k120_partial_wave", seg_rows=(6,), E=128, K=120, H=320, I=192,
              w_scales="pow2"),
    # the single-workgroup layout's limit: 4096 slots (four 1024-slot chunks) and just past
    # it (the three-kernel layout), on a partial expert range
    wl.scaled(C["ep8_share"], "layout_4096_slots", seg_rows=(300, 212), E=32, K=8, H=128, I=64,
              e_begin=8, e_end=24),
    wl.scaled(C["ep8_share"], "layout_4104_slots", seg_rows=(300, 213), E=32, K=8, H=128, I=64,
              e_begin=8, e_end=24),
    # degenerate shapes: one expert (every gate 1), one token, empty source segments
    wl.scaled(C["dsv3_prefill"], "single_expert", seg_rows=(37,), E=1, K=1, H=128, I=64),
    wl.scaled(C["dsv3_decode"], "single_token", seg_rows=(1,), E=8, K=2, H=128, I=64),
    wl.scaled(C["ep8_share"], "empty_segments", seg_rows=(0, 7, 0, 0, 5, 0), E=16, K=3, H=128, I=64,
              e_begin=2, e_end=9),
]


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def check_exact_stages(g, o, act):
    np.testing.assert_array_equal(g["ids"], o["ids"])
    np.testing.assert_allclose(g["gates"], o["gates"], rtol=1e-5, atol=1e-7)
    np.testing.assert_array_equal(g["counts"], o["counts"])
    np.testing.assert_array_equal(g["offsets"], o["offsets"])
    np.testing.assert_array_equal(g["row_of"], o["row_of"])
    np.testing.assert_array_equal(g["src_of"], o["src_of"])
    R = g["R"]
    np.testing.assert_array_equal(g["xd"], o["xd"][:R])
    if act == "fp8":
        np.testing.assert_array_equal(g["xd_scales"], o["xd_scales"][:R])


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_layer_parity_small(cfg):
    print(f"[parity] {cfg.name} T={cfg.T} E={cfg.E} K={cfg.K} H={cfg.H} I={cfg.I}", flush=True)
    case = Case(cfg)
    layer = run_gpu(case)
    g = gpu_view(layer)
    o = case.oracle_layer()
    check_exact_stages(g, o, cfg.act_dtype)
    assert_close(g["y"], o["y"], cfg.act_dtype, "y")
    assert_close(g["out"], o["out"], cfg.act_dtype, "out")
    del case, layer
    _free()


def _forced_case(cfg, logits):
    case = Case(cfg)
    case.logits_cpu = torch.as_tensor(logits, dtype=torch.float32)
    case.logits_dev = case.logits_cpu.cuda()
    return case


@pytest.mark.parametrize("act,T", [("bf16", 300), ("bf16", 600), ("fp8", 40), ("fp8", 300), ("fp8", 600)])
def test_all_tokens_one_expert_rest_empty(act, T):
    """All rows on one expert (several m-tiles of the 128-row and of the
    256-row kernels, split evenly; for fp8 at T = 40 the 16-row tiles with
    staged weight-scale bytes, at T = 600 the 192-row wide tiles), seven
    experts empty."""
    base = C["dsv3_prefill"] if act == "bf16" else C["gptoss_fp8"]
    cfg = wl.scaled(base, f"one_expert_{act}_{T}", seg_rows=(T,), E=8, K=1, H=256, I=192)
    lg = np.random.default_rng(0).normal(size=(T, 8)).astype(np.float32)
    lg[:, 5] += 100.0                      # every token picks expert 5, 7 experts stay empty
    case = _forced_case(cfg, lg)
    g = gpu_view(run_gpu(case))
    o = case.oracle_layer()
    assert o["counts"][5] == T and (o["counts"] == 0).sum() == 7
    check_exact_stages(g, o, act)
    assert_close(g["y"], o["y"], act, "y")
    assert_close(g["out"], o["out"], act, "out")


def test_k_equals_e_and_ties():
    cfg = wl.scaled(C["dsv3_prefill"], "k_eq_e", seg_rows=(50,), E=4, K=4, H=128, I=64)
    lg = np.random.default_rng(1).integers(-1, 2, size=(50, 4)).astype(np.float32)
    case = _forced_case(cfg, lg)
    g = gpu_view(run_gpu(case))
    o = case.oracle_layer()
    check_exact_stages(g, o, "bf16")
    assert_close(g["out"], o["out"], "bf16", "out")


def test_route_ties_and_negative_zero():
    from combine_grouped_gemm_amd import moe_route
    rng = np.random.default_rng(2)
    for E, K in ((16, 2), (64, 8), (256, 8), (200, 17), (1024, 5), (7, 7)):
        lg = rng.integers(-1, 2, size=(257, E)).astype(np.float32)
        lg[0, :] = 0.0
        lg[1, ::2] = -0.0
        ids, w = moe_route(torch.from_numpy(lg).cuda(), K)
        oi, ow = oracle.route(lg, K)
        np.testing.assert_array_equal(ids.cpu().numpy(), oi)
        np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=1e-5, atol=1e-7)


def test_empty_batch():
    cfg = wl.scaled(C["dsv3_prefill"], "empty", seg_rows=(0,), E=8, K=2, H=128, I=64)
    from combine_grouped_gemm_amd import MoELayer
    layer = MoELayer(cfg.seg_rows, cfg.E, cfg.K, cfg.H, cfg.I, 0, cfg.E, "bf16", "bf16", "bf16")
    x = [torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")]
    lg = torch.empty((0, cfg.E), dtype=torch.float32, device="cuda")
    w = wl.gen_expert_weights(cfg, "cuda")
    layer.forward(x, lg, {"gate": w.gate, "up": w.up, "down": w.down})
    torch.cuda.synchronize()
    assert layer.counts.cpu().sum() == 0 and int(layer.offsets[-1]) == 0


def test_capacity_overflow_drops_late_rows():
    """cap_rows below the routed rows: the first cap rows are the oracle's,
    later slots get row -1, and every kernel stays within the buffers."""
    cfg = wl.scaled(C["dsv3_prefill"], "overflow", seg_rows=(64,), E=4, K=2, H=128, I=64)
    case = Case(cfg)
    from combine_grouped_gemm_amd import MoELayer
    cap = 50
    layer = MoELayer(cfg.seg_rows, cfg.E, cfg.K, cfg.H, cfg.I, 0, cfg.E, "bf16", "bf16", "bf16",
                     cap_rows=cap)
    run_gpu(case, layer)
    o = oracle.layout(oracle.route(case.logits_np(), cfg.K)[0], cfg.E, 0, cfg.E, cfg.T * cfg.K)
    np.testing.assert_array_equal(layer.src_of.cpu().numpy(), o["src_of"][:cap])
    ro = layer.row_of.cpu().numpy()
    np.testing.assert_array_equal(ro, np.where(o["row_of"] < cap, o["row_of"], -1))
    np.testing.assert_array_equal(layer.offsets.cpu().numpy(), o["offsets"])


def test_fp8_grouped_call_matches_stage_calls():
    """moe_grouped_ffn carves h and its scales out of the workspace; the result
    must be bit-identical to the two stage calls with separate buffers."""
    from combine_grouped_gemm_amd import moe_grouped_ffn
    cfg = wl.scaled(C["gptoss_fp8"], "fp8_grouped", seg_rows=(256,), E=8, K=2, H=320, I=192)
    case = Case(cfg)
    layer = run_gpu(case)
    w = case.wdict
    y2 = moe_grouped_ffn(layer.xd, layer.xd_scales, layer.offsets, w["gate"], w["up"], w["down"],
                         w["gate_scale"], w["up_scale"], w["down_scale"],
                         expected_rows=layer.expected_rows, w_scales_pow2=w["scales_pow2"])
    torch.cuda.synchronize()
    R = int(layer.offsets[-1])
    assert torch.equal(y2[:R], layer.y[:R])


def test_fp8_pow2_weight_path_matches_generic_path():
    """Power-of-two weight scales declared (MOE_FP8_E4M3_PO2: every scale
    applied by the matrix cores) or not (weight scale folded in fp32 per
    block product): the same numbers up to fp32 rounding order, so y agrees
    far inside the fp8 tolerance and h codes differ only where a value sits
    on a rounding boundary."""
    from combine_grouped_gemm_amd import moe_ffn_down, moe_ffn_gate_up
    cfg = wl.scaled(C["gptoss_fp8"], "fp8_po2_vs_generic", seg_rows=(600,), E=8, K=2, H=640, I=384,
                    w_scales="pow2")
    case = Case(cfg)
    assert case.w.scales_pow2
    layer = run_gpu(case)
    w = case.wdict
    kw = dict(expected_rows=layer.expected_rows)
    res = {}
    for po2 in (True, False):
        h, hs = moe_ffn_gate_up(layer.xd, layer.xd_scales, layer.offsets, w["gate"], w["up"],
                                w["gate_scale"], w["up_scale"], w_scales_pow2=po2, **kw)
        y = moe_ffn_down(h, hs, layer.offsets, w["down"], w["down_scale"], w_scales_pow2=po2, **kw)
        torch.cuda.synchronize()
        res[po2] = (h, hs, y)
    R = int(layer.offsets[-1])
    assert torch.equal(res[True][2][:R], layer.y[:R])          # the layer took the PO2 path
    codes_t = res[True][0][:R].view(torch.uint8)
    codes_f = res[False][0][:R].view(torch.uint8)
    assert (codes_t != codes_f).float().mean().item() < 1e-2
    yt, yf = res[True][2][:R].double(), res[False][2][:R].double()
    assert ((yt - yf).norm() / yf.norm()).item() < 1e-2


def test_deterministic_and_stage_split_matches_grouped_call():
    from combine_grouped_gemm_amd import moe_grouped_ffn
    cfg = wl.scaled(C["dsv3_prefill"], "det", seg_rows=(400,), E=8, K=2, H=256, I=192)
    case = Case(cfg)
    l1 = run_gpu(case)
    a = {k: v.clone() for k, v in (("y", l1.y), ("out", l1.out), ("xd", l1.xd))}
    run_gpu(case, l1)
    assert torch.equal(a["out"], l1.out) and torch.equal(a["y"], l1.y)
    y2 = moe_grouped_ffn(l1.xd, None, l1.offsets, case.w.gate, case.w.up, case.w.down)
    torch.cuda.synchronize()
    R = int(l1.offsets[-1])
    assert torch.equal(y2[:R], l1.y[:R])


# ----------------------------------------------------------------------------
# full workload sizes: exact checks on everything integer, sampled FP checks
# ----------------------------------------------------------------------------
FULL = ["dsv3_decode", "dsv3_prefill", "ep8_share", "gptoss_fp8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    cfg = C[name]
    print(f"[parity-full] {name} T={cfg.T}", flush=True)
    case = Case(cfg)
    layer = run_gpu(case)
    lg = case.logits_np()
    ids, gates = oracle.route(lg, cfg.K)
    np.testing.assert_array_equal(layer.topk_ids.cpu().numpy(), ids)
    np.testing.assert_allclose(layer.topk_w.cpu().numpy(), gates, rtol=1e-5, atol=1e-7)
    lay = oracle.layout(ids, cfg.E, cfg.e_begin, cfg.e_end, cfg.cap)
    for k in ("counts", "offsets", "row_of"):
        np.testing.assert_array_equal(getattr(layer, k).cpu().numpy(), lay[k])
    np.testing.assert_array_equal(layer.src_of.cpu().numpy(), lay["src_of"])
    R = int(lay["offsets"][-1])
    x = case.x_np()
    rng = np.random.default_rng(cfg.seed)
    # dispatch: sampled rows, exact
    rows = rng.choice(R, size=min(R, 64), replace=False)
    toks = lay["src_of"][rows] // cfg.K
    ox, oxs = oracle.dispatch(x[toks], np.arange(len(rows))[:, None], len(rows), cfg.act_dtype)
    np.testing.assert_array_equal(to_np(layer.xd[torch.as_tensor(rows).cuda()]), ox)
    if cfg.act_dtype == "fp8":
        np.testing.assert_array_equal(layer.xd_scales[torch.as_tensor(rows).cuda()].cpu().numpy(), oxs)
    # expert outputs: all rows of the busiest and of the least busy non-empty local
    # expert, and of three random ones
    off = lay["offsets"]
    n_rows = np.diff(off)
    busiest = int(np.argmax(n_rows))
    quietest = int(np.argmin(np.where(n_rows > 0, n_rows, np.iinfo(np.int64).max)))
    for j in sorted({busiest, quietest, *(int(v) for v in rng.choice(cfg.E_loc, size=3, replace=False))}):
        a, b = int(off[j]), int(off[j + 1])
        if b == a:
            continue
        xd_o, xs_o = oracle.dispatch(x[lay["src_of"][a:b] // cfg.K],
                                     np.arange(b - a)[:, None], b - a, cfg.act_dtype)
        xv = oracle.numerics.dequantize_fp8_blocks(xd_o, xs_o) if cfg.act_dtype == "fp8" else xd_o
        y_o = oracle.expert_ffn(xv, *case.oracle_weights(j), cfg.act_dtype, cfg.y_dtype)
        assert_close(to_np(layer.y[a:b]), y_o, cfg.act_dtype, f"y of local expert {j}")
    # combined rows of six tokens
    for t in rng.choice(cfg.T, size=6, replace=False):
        acc = np.zeros(cfg.H)
        xv_t, xs_t = oracle.dispatch(x[t:t + 1], np.zeros((1, 1), np.int64), 1, cfg.act_dtype)
        xv_t = oracle.numerics.dequantize_fp8_blocks(xv_t, xs_t) if cfg.act_dtype == "fp8" else xv_t
        for k in range(cfg.K):
            e = int(ids[t, k])
            if cfg.e_begin <= e < cfg.e_end:
                yk = oracle.expert_ffn(xv_t, *case.oracle_weights(e - cfg.e_begin),
                                       cfg.act_dtype, cfg.y_dtype)[0]
                acc += np.float64(np.float32(gates[t, k])) * yk
        ref = oracle.numerics.round_act(acc, cfg.out_dtype)
        assert_close(to_np(layer.out[int(t)]), ref, cfg.act_dtype, f"out[{t}]")
    # the bench feeds the weights packed to the padded row pitch: at full size
    # that layer gives the same bits as the one checked above
    import combine_grouped_gemm_amd as m
    y0, out0 = layer.y[:R].clone(), layer.out.clone()
    pk = dict(case.wdict)
    for k in ("gate", "up", "down"):
        pk[k] = m.moe_pack_weights(case.wdict[k])
    layer.forward(case.x_dev, case.logits_dev, pk)
    torch.cuda.synchronize()
    assert torch.equal(layer.y[:R].contiguous().view(torch.uint8), y0.contiguous().view(torch.uint8)), "y (packed)"
    assert torch.equal(layer.out.contiguous().view(torch.uint8), out0.contiguous().view(torch.uint8)), "out (packed)"
    del case, layer, pk, y0, out0
    _free()
