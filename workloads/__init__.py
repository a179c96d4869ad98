"""Seeded synthetic workloads for the MoE layer (shared by tests, bench and
smoke checks).

This module only draws random inputs; it holds none of the layer's arithmetic
(no top-K, no grouping, no GEMM, no activation quantisation).  fp8 expert
weights are prepared here as an fp8 checkpoint would ship them (codes plus
block scales, see gen_expert_weights): an input, not a step of the layer.
The router projection that produces the logits is the layer's input stage
and is computed here with a plain torch matmul, outside the timed path, so
that the oracle and the HIP path receive the very same logits tensor.

Workloads (shapes follow the pages: the toy EP layer of "Anatomy of a
high-performance EP kernel", section "What we have to do"; the 256-expert,
top-8 DeepSeek layer and the 32-experts-per-GPU split of the Moreh report,
"Parallelisation method"; a GPT-OSS-120B-shaped layer named in its
"Overview"):

  toy          8 ranks x 8 tokens, E=16, K=2, H=128, I=256, all fp32
  dsv3_decode  T=128, E=256, K=8, H=7168, I=2048, bf16
  dsv3_prefill T=8192, same layer
  ep8_share    8 source segments, B_i ~ U{256..768}, same layer, per-expert
               Zipf-shaped logit bias, local experts 0-31 of 256
  gptoss_fp8   T=4096, E=128, K=4, H=I=2880, fp8 e4m3 weights and
               dispatched activations with 1x128 fp32 block scales
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass, field, replace

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
FP8_BLOCK = 128


@dataclass(frozen=True)
class MoEConfig:
    name: str
    seg_rows: tuple          # tokens per simulated source rank
    E: int                   # routed experts
    K: int                   # experts per token
    H: int                   # hidden size
    I: int                   # expert intermediate size
    e_begin: int             # first local expert
    e_end: int               # one past the last local expert
    x_dtype: str             # 'f32' | 'bf16'
    act_dtype: str           # storage of Xd and h: 'f32' | 'bf16' | 'fp8'
    w_dtype: str             # 'f32' | 'bf16' | 'fp8'
    y_dtype: str             # 'f32' | 'bf16'
    out_dtype: str           # 'f32' | 'bf16'
    seed: int
    zipf_bias: bool = False
    description: str = ""
    w_scales: str = "fp32"   # fp8 weight block scales: 'fp32' (any positive value) | 'pow2'

    @property
    def T(self) -> int:
        return int(sum(self.seg_rows))

    @property
    def E_loc(self) -> int:
        return self.e_end - self.e_begin

    @property
    def cap(self) -> int:
        return self.T * self.K


def _draw_segments(seed: int, n: int, lo: int, hi: int) -> tuple:
    g = torch.Generator().manual_seed(seed * 1000 + 7)
    return tuple(int(v) for v in torch.randint(lo, hi + 1, (n,), generator=g))


CONFIGS = {
    "toy": MoEConfig("toy", (8,) * 8, 16, 2, 128, 256, 0, 16,
                     "f32", "f32", "f32", "f32", "f32", seed=1,
                     description="toy EP layer: 8 ranks x 8 tokens, E=16, K=2, fp32"),
    "dsv3_decode": MoEConfig("dsv3_decode", (128,), 256, 8, 7168, 2048, 0, 256,
                             "bf16", "bf16", "bf16", "bf16", "bf16", seed=2,
                             description="DeepSeek-V3-shaped decode step, T=128, bf16"),
    "dsv3_prefill": MoEConfig("dsv3_prefill", (8192,), 256, 8, 7168, 2048, 0, 256,
                              "bf16", "bf16", "bf16", "bf16", "bf16", seed=3,
                              description="DeepSeek-V3-shaped prefill, T=8192, bf16"),
    "ep8_share": MoEConfig("ep8_share", _draw_segments(4, 8, 256, 768), 256, 8, 7168, 2048,
                           0, 32, "bf16", "bf16", "bf16", "bf16", "bf16", seed=4,
                           zipf_bias=True,
                           description="one EP=8 rank's share: 8 segments, local experts 0-31, "
                                       "Zipf-biased routing"),
    "gptoss_fp8": MoEConfig("gptoss_fp8", (4096,), 128, 4, 2880, 2880, 0, 128,
                            "bf16", "fp8", "fp8", "bf16", "bf16", seed=5,
                            description="GPT-OSS-120B-shaped layer, fp8 e4m3 weights and "
                                        "activations with 1x128 fp32 block scales",
                            w_scales="fp32"),
}


def scaled(cfg: MoEConfig, name: str, *, seg_rows=None, E=None, K=None, H=None, I=None,
           e_begin=None, e_end=None, seed=None, w_scales=None) -> MoEConfig:
    """A smaller (or otherwise changed) copy of a workload, for parity tests."""
    E = cfg.E if E is None else E
    kw = dict(name=name,
              seg_rows=cfg.seg_rows if seg_rows is None else tuple(seg_rows),
              E=E, K=cfg.K if K is None else K, H=cfg.H if H is None else H,
              I=cfg.I if I is None else I,
              e_begin=0 if e_begin is None else e_begin,
              e_end=E if e_end is None else e_end,
              seed=cfg.seed if seed is None else seed,
              w_scales=cfg.w_scales if w_scales is None else w_scales,
              zipf_bias=False)           # the calibrated bias belongs to the named workload only
    return replace(cfg, **kw)


# ----------------------------------------------------------------------------
# token activations and logits (CPU, torch generator)
# ----------------------------------------------------------------------------
def _storage(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def gen_x(cfg: MoEConfig) -> list:
    """One CPU tensor (B_i, H) per source segment, x ~ N(0, 1) stored as x_dtype."""
    g = torch.Generator().manual_seed(cfg.seed * 1000 + 11)
    out = []
    for b in cfg.seg_rows:
        out.append(torch.randn(b, cfg.H, generator=g).to(_storage(cfg.x_dtype)))
    return out


def gen_router(cfg: MoEConfig) -> torch.Tensor:
    """Router weight W_r (E, H) fp32, N(0, 1/H)."""
    g = torch.Generator().manual_seed(cfg.seed * 1000 + 13)
    return torch.randn(cfg.E, cfg.H, generator=g) / math.sqrt(cfg.H)


def zipf_bias_params(cfg: MoEConfig):
    """(beta, shift) for the per-expert logit bias, as stored by the
    calibration script beside this module; None if the workload has none."""
    if not cfg.zipf_bias:
        return None
    with open(os.path.join(_HERE, "zipf_bias.json")) as f:
        d = json.load(f)
    return float(d[cfg.name]["beta"]), int(d[cfg.name]["shift"])


def zipf_bias(cfg: MoEConfig, beta: float, shift: int) -> torch.Tensor:
    """bias_e = beta * ln(z_e) with z_e = pi(e)^-1.1 for a seeded permutation
    pi of 1..E, rotated by ``shift`` experts.  fp32 (E,)."""
    g = torch.Generator().manual_seed(cfg.seed * 1000 + 17)
    pi = torch.randperm(cfg.E, generator=g).double() + 1.0
    pi = torch.roll(pi, -shift)
    return (beta * (-1.1) * torch.log(pi)).float()


def gen_logits(cfg: MoEConfig, x_segments=None, bias_params=None) -> torch.Tensor:
    """Router logits (T, E) fp32 = x W_r^T (+ bias), x taken segment-major.

    ``bias_params`` overrides the stored (beta, shift) (the calibration script
    uses it); pass ``False`` for no bias."""
    if x_segments is None:
        x_segments = gen_x(cfg)
    x = torch.cat([s.float() for s in x_segments], dim=0)
    logits = x @ gen_router(cfg).T
    if bias_params is None:
        bias_params = zipf_bias_params(cfg)
    if bias_params:
        logits = logits + zipf_bias(cfg, *bias_params)[None, :]
    return logits.contiguous()


def gen_calibration_logits(cfg: MoEConfig, seed_offset: int = 1000, batches: int = 1) -> torch.Tensor:
    """Router logits of other batches of the same model: ``batches`` batches
    of the workload's size, tokens drawn with seeds seed + seed_offset + b,
    the workload's own router weights and logit bias.  Expert activation
    counts measured on them drive expert placement."""
    w_r = gen_router(cfg)
    bias_params = zipf_bias_params(cfg)
    bias = zipf_bias(cfg, *bias_params)[None, :] if bias_params else None
    out = []
    for b in range(batches):
        other = replace(cfg, seed=cfg.seed + seed_offset + b)
        x = torch.cat([s.float() for s in gen_x(other)], dim=0)
        lg = x @ w_r.T
        out.append(lg + bias if bias is not None else lg)
        del x
    return torch.cat(out, dim=0).contiguous()


# ----------------------------------------------------------------------------
# expert weights
# ----------------------------------------------------------------------------
@dataclass
class ExpertWeights:
    """Local expert weights in the logical (out, in) layout.

    gate, up: (E_loc, I, H); down: (E_loc, H, I).  For fp8 these hold the
    e4m3 codes (torch.float8_e4m3fn) and *_scale the fp32 block scales with
    shapes (E_loc, I, ceil(H/128)) and (E_loc, H, ceil(I/128))."""
    gate: torch.Tensor
    up: torch.Tensor
    down: torch.Tensor
    gate_scale: torch.Tensor = None
    up_scale: torch.Tensor = None
    down_scale: torch.Tensor = None
    dtype: str = "bf16"
    scales_pow2: bool = False      # fp8: every block scale is a power of two

    def as_dict(self) -> dict:
        """The tensors as the layer takes them (no copies)."""
        d = {"gate": self.gate, "up": self.up, "down": self.down}
        if self.dtype == "fp8":
            d.update(gate_scale=self.gate_scale, up_scale=self.up_scale,
                     down_scale=self.down_scale, scales_pow2=self.scales_pow2)
        return d

    def expert(self, e: int, device="cpu") -> dict:
        """Copies of local expert e's tensors on ``device``."""
        d = {"gate": self.gate[e].to(device), "up": self.up[e].to(device),
             "down": self.down[e].to(device)}
        if self.dtype == "fp8":
            d.update(gate_scale=self.gate_scale[e].to(device),
                     up_scale=self.up_scale[e].to(device),
                     down_scale=self.down_scale[e].to(device))
        return d


def _expert_generator(cfg: MoEConfig, e_global: int, which: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed * 1_000_003 + e_global * 7 + which)
    return g


def _draw_fp32(cfg: MoEConfig, e_global: int, which: int, shape, device) -> torch.Tensor:
    """Matrix `which` (0 gate, 1 up, 2 down) of expert e_global, fp32
    N(0, 1/fan_in) with fan_in = shape[1]."""
    g = _expert_generator(cfg, e_global, which, device)
    return torch.randn(shape, generator=g, device=device) / math.sqrt(shape[1])


def gen_expert_weights_fp32(cfg: MoEConfig, device="cpu", experts=None) -> ExpertWeights:
    """The fp32 weights an fp8 workload's codes and scales are quantised from
    (the same draws as gen_expert_weights), for measuring what quantisation
    costs.  gate, up (E_loc, I, H); down (E_loc, H, I)."""
    experts = list(range(cfg.e_begin, cfg.e_end)) if experts is None else [int(e) for e in experts]
    shapes = ((cfg.I, cfg.H), (cfg.I, cfg.H), (cfg.H, cfg.I))
    mats = [torch.stack([_draw_fp32(cfg, e, w, s, device) for e in experts]) for w, s in enumerate(shapes)]
    return ExpertWeights(*mats, dtype="f32")


def gen_expert_weights(cfg: MoEConfig, device="cpu", experts=None) -> ExpertWeights:
    """Expert weights drawn on ``device``, N(0, 1/fan_in) in value.

    ``experts`` lists the (logical) expert of each local slot; default the
    local range [e_begin, e_end).  A placement that renumbers experts passes
    the logical expert held by each local physical slot.

    Each (expert, matrix) pair has its own seeded generator, so a workload's
    weights are the same whichever subset of experts is drawn, but they
    depend on the device's generator (CPU and GPU streams differ).

    fp8 weights are fp32 weights ~ N(0, 1/fan_in) stored the way an fp8
    checkpoint ships them: per output row, one fp32 scale per block of 128
    input columns (the last block narrower when fan_in is not a multiple of
    128), s = amax / 448 over the block (1 for an all-zero block), and codes
    = the e4m3 cast of w / s (torch's conversion, the values clamped to
    +-448 first).  With cfg.w_scales == 'pow2' each scale is instead the
    smallest power of two with amax <= 448 * s.  This prepares the inputs
    only: the layer receives codes and scales, and its own quantisation of
    activations is defined elsewhere.
    """
    experts = list(range(cfg.e_begin, cfg.e_end)) if experts is None else [int(e) for e in experts]
    E_loc, H, I = len(experts), cfg.H, cfg.I
    shapes = ((I, H), (I, H), (H, I))
    if cfg.w_dtype in ("f32", "bf16"):
        dt = _storage(cfg.w_dtype)
        mats = [torch.empty((E_loc,) + s, dtype=dt, device=device) for s in shapes]
        for j, e in enumerate(experts):
            for w, (m, s) in enumerate(zip(mats, shapes)):
                g = _expert_generator(cfg, e, w, device)
                m[j].copy_((torch.randn(s, generator=g, device=device) / math.sqrt(s[1])).to(dt))
        return ExpertWeights(*mats, dtype=cfg.w_dtype)
    if cfg.w_dtype == "fp8":
        codes, scales = [], []
        for s in shapes:
            nb = -(-s[1] // FP8_BLOCK)
            codes.append(torch.empty((E_loc,) + s, dtype=torch.float8_e4m3fn, device=device))
            scales.append(torch.empty((E_loc, s[0], nb), dtype=torch.float32, device=device))
        for j, e in enumerate(experts):
            for w, s in enumerate(shapes):
                wf = _draw_fp32(cfg, e, w, s, device)
                nb = scales[w].shape[2]
                pad = nb * FP8_BLOCK - s[1]
                amax = torch.nn.functional.pad(wf.abs(), (0, pad)).view(s[0], nb, FP8_BLOCK).amax(dim=2)
                sc = amax / 448.0
                if cfg.w_scales == "pow2":
                    m, ex = torch.frexp(sc)                  # sc = m * 2^ex, m in [0.5, 1)
                    sc = torch.ldexp(torch.ones_like(sc), torch.where(m == 0.5, ex - 1, ex))
                sc = torch.where(amax > 0, sc, torch.ones_like(sc))
                full = sc.repeat_interleave(FP8_BLOCK, dim=1)[:, :s[1]]
                codes[w][j].copy_((wf / full).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn))
                scales[w][j].copy_(sc)
        return ExpertWeights(codes[0], codes[1], codes[2], scales[0], scales[1], scales[2],
                             dtype="fp8", scales_pow2=cfg.w_scales == "pow2")
    raise ValueError(cfg.w_dtype)
