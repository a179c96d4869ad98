"""What the fp8 activation-scale rule costs in precision: the GPT-OSS-shaped
layer computed by the oracle with fp8 activations under two block-scale
rules, each compared with the same layer computed without any fp8 rounding.

Test infrastructure only (calls nothing but ``oracle`` and the seeded input
generators).  The pages name block-wise fp8 quantisation for the grouped GEMM
(SGLang "Expert Parallelism", the MoE backend table) without its scale rule;
the layer reads it as one power-of-two scale per 1x128 block (the E8M0
convention, applied exactly by the matrix cores).  The alternative rule,
s = amax / 448, puts each block's largest magnitude on the top e4m3 code.

    python -m oracle.fp8_scale_study [--tokens 256] [--experts 8]

Prints one JSON object: relative L2 errors of y and out for each rule, for
the workload's fp8 weights (fp32 block scales) and for the same weights with
power-of-two weight scales.  The reference keeps x in bf16 (the layer's
input), the fp32 weights the codes were quantised from, and every
intermediate in fp64.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import moe  # noqa: E402
from oracle import numerics as nx  # noqa: E402


def _ffn(X, Wg, Wu, Wd, act_rule):
    """One expert on rows X (values the expert sees): act_rule None keeps h
    in fp64, else h is block-quantised to fp8 with that rule; y in fp64."""
    g = X @ Wg.T
    u = X @ Wu.T
    h = moe.silu(g) * u
    if act_rule is not None:
        h = nx.dequantize_fp8_blocks(*nx.quantize_fp8_blocks(nx.to_f32(h), rule=act_rule))
    return h @ Wd.T


def run(tokens=256, experts=8):
    import torch  # noqa: F401  (the generators draw with torch)
    import workloads as wl
    base = wl.CONFIGS["gptoss_fp8"]
    cfg = wl.scaled(base, "fp8_scale_study", seg_rows=(tokens,), E=experts)
    x = np.concatenate([t.float().numpy().astype(np.float64) for t in wl.gen_x(cfg)])
    ids, gates = moe.route(wl.gen_logits(cfg).numpy(), cfg.K)
    gates = nx.to_f32(gates)
    lay = moe.layout(ids, cfg.E, 0, cfg.E, cfg.T * cfg.K)
    off, src = lay["offsets"], lay["src_of"]
    R = int(off[-1])
    w32 = wl.gen_expert_weights_fp32(cfg)
    ref_w = [tuple(t[j].double().numpy() for t in (w32.gate, w32.up, w32.down)) for j in range(cfg.E)]

    def fp8_weights(w_scales):
        W = wl.gen_expert_weights(wl.scaled(cfg, cfg.name, w_scales=w_scales))
        out = []
        for j in range(cfg.E):
            d = W.expert(j)
            out.append(tuple(nx.dequantize_fp8_blocks(d[k].float().numpy().astype(np.float64),
                                                      d[k + "_scale"].numpy())
                             for k in ("gate", "up", "down")))
        return out

    def layer(weights, act_rule):
        y = np.zeros((R, cfg.H))
        for j in range(cfg.E):
            a, b = int(off[j]), int(off[j + 1])
            X = x[src[a:b] // cfg.K]
            if act_rule is not None:
                X = nx.dequantize_fp8_blocks(*nx.quantize_fp8_blocks(X, rule=act_rule))
            y[a:b] = _ffn(X, *weights[j], act_rule)
        out = moe.combine(y, lay["row_of"], gates, "f32")
        return y, out

    y_ref, out_ref = layer(ref_w, None)

    def rel(a, b):
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))

    res = {"config": {"T": cfg.T, "E": cfg.E, "K": cfg.K, "H": cfg.H, "I": cfg.I, "rows": R},
           "reference": "x bf16, fp32 weights before quantisation, no fp8 rounding, fp64 arithmetic"}
    for w_scales in ("fp32", "pow2"):
        W = fp8_weights(w_scales)
        res[f"weights_{w_scales}_scales_only"] = {"y": rel(layer(W, None)[0], y_ref),
                                                   "out": rel(layer(W, None)[1], out_ref)}
        for rule in ("pow2", "amax448"):
            y, out = layer(W, rule)
            res[f"weights_{w_scales}_scales+activations_{rule}"] = {"y": rel(y, y_ref), "out": rel(out, out_ref)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--tokens", type=int, default=256)
    ap.add_argument("--experts", type=int, default=8)
    a = ap.parse_args()
    print(json.dumps(run(a.tokens, a.experts), indent=1))


if __name__ == "__main__":
    main()
