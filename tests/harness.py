"""Shared helpers of the parity tests: build a workload's inputs, run the HIP
path through the binding, and fetch tensors the oracle can read.

Expected values come only from ``oracle``; the HIP path's outputs are only
ever compared against them.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import numerics as nx
import workloads as wl


def has_gpu() -> bool:
    return torch.cuda.is_available()


def to_np(t: torch.Tensor) -> np.ndarray:
    """fp64 numpy copy of a (device or host) tensor's values."""
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float8_e4m3fn, torch.float16):
        t = t.float()
    return t.cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def rel_l2(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    d = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (d if d > 0 else 1.0))


def max_abs(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


# floating-point bars: bf16 and fp8 from the layer's stated tolerance; fp32
# tightened for an all-fp32 layer (fp32 accumulation over <= 256 terms of
# O(1) values, compared with fp64: relative error well below 1e-5)
TOL = {"bf16": dict(rel=1e-2, abs=5e-2), "fp8": dict(rel=3e-2, abs=None),
       "f32": dict(rel=1e-5, abs=1e-4)}


def assert_close(got, ref, act: str, what: str):
    t = TOL[act]
    r = rel_l2(got, ref)
    assert r <= t["rel"], f"{what}: relative L2 {r:.3e} > {t['rel']:.1e}"
    if t["abs"] is not None:
        m = max_abs(got, ref)
        assert m <= t["abs"], f"{what}: max-abs {m:.3e} > {t['abs']:.1e}"


class Case:
    """A workload's inputs on the device plus oracle views of them."""

    def __init__(self, cfg: wl.MoEConfig, device="cuda"):
        self.cfg = cfg
        self.x_cpu = wl.gen_x(cfg)
        self.logits_cpu = wl.gen_logits(cfg, self.x_cpu)
        self.x_dev = [s.to(device) for s in self.x_cpu]
        self.logits_dev = self.logits_cpu.to(device)
        self.w = wl.gen_expert_weights(cfg, device=device)
        self.wdict = self.w.as_dict()

    # oracle views --------------------------------------------------------------
    def x_np(self) -> np.ndarray:
        return np.concatenate([to_np(s) for s in self.x_cpu], axis=0)

    def logits_np(self) -> np.ndarray:
        return self.logits_cpu.numpy()

    def oracle_weights(self, j: int):
        """Dequantised fp64 (Wg, Wu, Wd) of local expert j."""
        d = self.w.expert(j, "cpu")
        if self.cfg.w_dtype == "fp8":
            return tuple(nx.dequantize_fp8_blocks(to_np(d[k]), to_np(d[k + "_scale"]))
                         for k in ("gate", "up", "down"))
        return tuple(to_np(d[k]) for k in ("gate", "up", "down"))

    def oracle_layer(self):
        c = self.cfg
        return oracle.layer(self.x_np(), self.logits_np(), c.K, c.E, c.e_begin, c.e_end,
                            self.oracle_weights, c.act_dtype, c.y_dtype, c.out_dtype)


def run_gpu(case: Case, layer=None):
    """Run the six library calls; return (layer, dict of host copies)."""
    from combine_grouped_gemm_amd import MoELayer
    c = case.cfg
    if layer is None:
        layer = MoELayer(c.seg_rows, c.E, c.K, c.H, c.I, c.e_begin, c.e_end, c.act_dtype,
                         c.y_dtype, c.out_dtype)
    layer.forward(case.x_dev, case.logits_dev, case.wdict)
    torch.cuda.synchronize()
    return layer


def gpu_view(layer) -> dict:
    R = int(layer.offsets[-1].item())
    v = {"ids": layer.topk_ids.cpu().numpy(), "gates": layer.topk_w.cpu().numpy(),
         "counts": layer.counts.cpu().numpy(), "offsets": layer.offsets.cpu().numpy(),
         "row_of": layer.row_of.cpu().numpy(), "src_of": layer.src_of.cpu().numpy()[:layer.cap],
         "R": R, "out": to_np(layer.out)}
    v["xd"] = to_np(layer.xd[:R])
    v["y"] = to_np(layer.y[:R])
    if layer.xd_scales is not None:
        v["xd_scales"] = layer.xd_scales[:R].cpu().numpy()
    return v
