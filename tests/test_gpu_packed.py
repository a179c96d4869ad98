"""Packed expert weights on the GPU.

moe_pack_weights must reproduce every row and zero the padding (bit-exact
against a padded copy made with torch), and every FFN kernel family fed
packed weights must give outputs bitwise identical to the same call on the
dense weights -- the layout changes only where a row starts, never the
arithmetic.  The dense path is itself held to the oracle in
test_gpu_parity.py; one packed layer per kernel family is also compared with
the oracle here.
"""
import gc

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import combine_grouped_gemm_amd as m
import workloads as wl
from harness import Case, assert_close, gpu_view, has_gpu, run_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

C = wl.CONFIGS

# (case, kernel family it lands on); dimensions chosen so that the packed
# pitch differs from the row length for at least one weight matrix
CASES = [
    # fp32: down rows of 1024 floats (4 KiB) -> pitch 1056
    (wl.scaled(C["toy"], "pk_f32", seg_rows=(24, 40), E=8, K=2, H=128, I=1024), "f32"),
    # bf16, ~5 rows per expert (16-row tiles): down rows 2048 bf16 (4 KiB) -> 2112
    (wl.scaled(C["dsv3_decode"], "pk_bf16_16row", seg_rows=(40,), E=32, K=4, H=256, I=2048), "bf16 16-row"),
    # bf16, ~37 rows per expert (128-row tiles)
    (wl.scaled(C["dsv3_decode"], "pk_bf16_128row", seg_rows=(300,), E=16, K=2, H=256, I=2048), "bf16 128-row"),
    # bf16, ~150 rows per expert (256-row wide tiles); gate/up rows 2048 too
    (wl.scaled(C["dsv3_prefill"], "pk_bf16_wide256", seg_rows=(600,), E=8, K=2, H=2048, I=2048), "bf16 wide 256"),
    # bf16, ~200 rows per expert (320-row wide tiles)
    (wl.scaled(C["dsv3_prefill"], "pk_bf16_wide320", seg_rows=(800,), E=4, K=1, H=2048, I=2048), "bf16 wide 320"),
    # fp8, ~15 rows per expert (register-staged tiles): 320 -> 384, 192 -> 256 bytes
    (wl.scaled(C["gptoss_fp8"], "pk_fp8_narrow", seg_rows=(60,), E=8, K=2, H=320, I=192, w_scales="fp32"), "fp8 narrow"),
    (wl.scaled(C["gptoss_fp8"], "pk_fp8_narrow_po2", seg_rows=(60,), E=8, K=2, H=320, I=192, w_scales="pow2"), "fp8 narrow"),
    # fp8 at H = I = 2880 (~50 rows per expert: the wide tiles): 2880 -> 2944 bytes
    (wl.scaled(C["gptoss_fp8"], "pk_fp8_wide", seg_rows=(200,), E=8, K=2, w_scales="fp32"), "fp8 wide"),
    (wl.scaled(C["gptoss_fp8"], "pk_fp8_wide_po2", seg_rows=(200,), E=8, K=2, w_scales="pow2"), "fp8 wide"),
]


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _bytes(t):
    return t.contiguous().view(torch.uint8)


def packed_dict(wd):
    out = dict(wd)
    for k in ("gate", "up", "down"):
        out[k] = m.moe_pack_weights(wd[k])
    return out


@pytest.mark.parametrize("dtype,cols", [(torch.float32, 1024), (torch.bfloat16, 2048), (torch.bfloat16, 7168),
                                        (torch.float8_e4m3fn, 2880), (torch.float8_e4m3fn, 4096),
                                        (torch.bfloat16, 72)])
def test_pack_reproduces_rows_and_zeroes_padding(dtype, cols):
    g = torch.Generator(device="cuda").manual_seed(cols)
    w = torch.randn((3, 37, cols), generator=g, device="cuda").to(dtype)
    ld = m.moe_weight_ld(cols, dtype)
    # stale bytes in the output must be overwritten: fill it first
    out = torch.full((3, 37, ld * w.element_size()), 7, dtype=torch.uint8, device="cuda").view(dtype)
    m.moe_pack_weights(w, out=out)
    ref = F.pad(_bytes(w).view(3, 37, -1), (0, (ld - cols) * w.element_size()))
    torch.cuda.synchronize()
    assert torch.equal(_bytes(out).view(3, 37, -1), ref)


@pytest.mark.parametrize("cfg,family", CASES, ids=[c.name for c, _ in CASES])
def test_packed_layer_bitwise_equals_dense(cfg, family):
    print(f"[packed] {cfg.name} ({family})", flush=True)
    case = Case(cfg)
    dense = run_gpu(case)
    want = {k: getattr(dense, k).clone() for k in ("h", "y", "out")}
    R = int(dense.offsets[-1].item())
    pk = packed_dict(case.wdict)
    assert any(pk[k].shape != case.wdict[k].shape for k in ("gate", "down")), "no padding exercised"
    layer = m.MoELayer(cfg.seg_rows, cfg.E, cfg.K, cfg.H, cfg.I, cfg.e_begin, cfg.e_end, cfg.act_dtype,
                       cfg.y_dtype, cfg.out_dtype)
    layer.forward(case.x_dev, case.logits_dev, pk)
    torch.cuda.synchronize()
    assert torch.equal(_bytes(layer.h[:R]), _bytes(want["h"][:R])), "h differs"
    if layer.h_scales is not None:
        assert torch.equal(layer.h_scales[:R], dense.h_scales[:R]), "h scales differ"
    assert torch.equal(_bytes(layer.y[:R]), _bytes(want["y"][:R])), "y differs"
    assert torch.equal(_bytes(layer.out), _bytes(want["out"])), "out differs"
    del dense, layer, pk, case
    _free()


@pytest.mark.parametrize("cfg,family", [CASES[0], CASES[3], CASES[7]], ids=["f32", "bf16_wide", "fp8_wide"])
def test_packed_layer_matches_oracle(cfg, family):
    case = Case(cfg)
    layer = m.MoELayer(cfg.seg_rows, cfg.E, cfg.K, cfg.H, cfg.I, cfg.e_begin, cfg.e_end, cfg.act_dtype,
                       cfg.y_dtype, cfg.out_dtype)
    layer.forward(case.x_dev, case.logits_dev, packed_dict(case.wdict))
    torch.cuda.synchronize()
    g = gpu_view(layer)
    o = case.oracle_layer()
    np.testing.assert_array_equal(g["row_of"], o["row_of"])
    assert_close(g["out"], o["out"], cfg.act_dtype, f"{cfg.name} out")
    del layer, case
    _free()


@pytest.mark.parametrize("act", ["bf16", "fp8"])
def test_packed_masked_ffn_bitwise_equals_dense(act):
    """The masked-layout FFN calls read packed weights the same way."""
    E_loc, cap_e, H, I = 4, 80, 256, 2048 if act == "bf16" else 2880
    if act == "fp8":
        H = 2880
    g = torch.Generator(device="cuda").manual_seed(11)
    dt = torch.bfloat16 if act == "bf16" else torch.float8_e4m3fn
    xd = (torch.randn((E_loc * cap_e, H), generator=g, device="cuda") * 0.5).to(dt)
    wg = (torch.randn((E_loc, I, H), generator=g, device="cuda") * 0.05).to(dt)
    wu = (torch.randn((E_loc, I, H), generator=g, device="cuda") * 0.05).to(dt)
    wd = (torch.randn((E_loc, H, I), generator=g, device="cuda") * 0.05).to(dt)
    mm = torch.tensor([80, 0, 33, 79], dtype=torch.int32, device="cuda")
    kw = {}
    if act == "fp8":
        nbH, nbI = -(-H // 128), -(-I // 128)
        xs = torch.full((E_loc * cap_e, nbH), 2.0 ** -3, device="cuda")
        kw = dict(w_gate_scales=torch.full((E_loc, I, nbH), 0.01, device="cuda"),
                  w_up_scales=torch.full((E_loc, I, nbH), 0.02, device="cuda"))
        kd = dict(w_down_scales=torch.full((E_loc, H, nbI), 0.015, device="cuda"))
    else:
        xs, kd = None, {}
    h0, hs0 = m.moe_ffn_gate_up_masked(xd, xs, mm, cap_e, wg, wu, **kw)
    y0 = m.moe_ffn_down_masked(h0, hs0, mm, cap_e, wd, **kd)
    h1, hs1 = m.moe_ffn_gate_up_masked(xd, xs, mm, cap_e, m.moe_pack_weights(wg), m.moe_pack_weights(wu), **kw)
    y1 = m.moe_ffn_down_masked(h1, hs1, mm, cap_e, m.moe_pack_weights(wd), **kd)
    torch.cuda.synchronize()
    for j, cnt in enumerate(mm.tolist()):
        r0, r1 = j * cap_e, j * cap_e + cnt
        assert torch.equal(_bytes(h1[r0:r1]), _bytes(h0[r0:r1])), f"h of expert {j}"
        assert torch.equal(_bytes(y1[r0:r1]), _bytes(y0[r0:r1])), f"y of expert {j}"
        if hs0 is not None:
            assert torch.equal(hs1[r0:r1], hs0[r0:r1])


def test_packed_and_dense_weights_cannot_mix():
    cfg = wl.scaled(C["dsv3_decode"], "pk_mix", seg_rows=(16,), E=4, K=2, H=2048, I=2048)
    case = Case(cfg)
    wd = dict(case.wdict)
    wd["down"] = m.moe_pack_weights(wd["down"])
    wd["gate"] = m.moe_pack_weights(wd["gate"])
    xd = torch.zeros((32, 2048), dtype=torch.bfloat16, device="cuda")
    offs = torch.zeros(5, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="w_up must have shape"):
        m.moe_grouped_ffn(xd, None, offs, wd["gate"], case.wdict["up"], wd["down"])
    with pytest.raises(ValueError, match="all packed or all dense"):
        m.moe_grouped_ffn(xd, None, offs, case.wdict["gate"], case.wdict["up"], wd["down"])
    with pytest.raises(ValueError, match="columns"):
        m.moe_ffn_down(xd[:, :2048], None, offs, wd["down"][:, :, :2100].contiguous())
