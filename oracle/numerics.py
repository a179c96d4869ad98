"""Number formats used by the MoE layer oracle: bf16, OCP fp8 e4m3fn, fp32.

Test infrastructure only: nothing under ``oracle/`` is part of the product path.

The formats themselves are not defined on the pages.  The SGLang "Expert
Parallelism" page (backend table for MoE computation, the DeepGEMM row) names
block-wise fp8 quantisation for the grouped GEMM; the convention used here
(OCP e4m3fn, one fp32 scale per 1x128 block along the contraction dimension;
for activations the scale is the smallest power of two s with amax / s <= 448,
the E8M0 convention of the microscaling formats; round to nearest even,
saturate at +-448) is a reading that both sides implement, so its geometry is
"parity unpinned" as far as the pages go.  Weight scales are arbitrary fp32
values given with the weights.  The rounding helpers themselves are pinned against torch's CPU casts.

Every function rounds from exact fp64 values by the definition of a binary
floating-point grid: scale the value so that one unit in the last place is 1,
round to the nearest integer with ties to even, scale back.
"""
from __future__ import annotations

import numpy as np

# --- format parameters: significand bits p (implicit bit included), minimum
# normal exponent, largest finite magnitude.
BF16_P, BF16_EMIN, BF16_MAX = 8, -126, float((2.0 - 2.0**-7) * 2.0**127)
E4M3_P, E4M3_EMIN, E4M3_MAX = 4, -6, 448.0
FP8_BLOCK = 128


def round_to_grid(v, p: int, emin: int) -> np.ndarray:
    """Round fp64 values to the nearest point of a binary grid with ``p``
    significand bits and minimum normal exponent ``emin`` (gradual underflow
    below it), ties to even.  No overflow handling: callers decide."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                    # v = m * 2**e with 0.5 <= |m| < 1
    lead = np.maximum(e - 1, emin)        # exponent of the leading bit
    q = lead - (p - 1)                    # exponent of one ulp
    return np.ldexp(np.rint(np.ldexp(v, -q)), q)   # np.rint: half to even


def to_bf16(v) -> np.ndarray:
    """Nearest bf16 value (RNE) of each element, returned as fp64.
    Magnitudes that round past the largest finite bf16 become +-inf."""
    r = round_to_grid(v, BF16_P, BF16_EMIN)
    return np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)


def to_f32(v) -> np.ndarray:
    """Nearest fp32 value (RNE) of each element, returned as fp64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def to_e4m3_sat(v) -> np.ndarray:
    """Nearest e4m3fn value (RNE) after clamping to [-448, 448], as fp64."""
    c = np.clip(np.asarray(v, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    return round_to_grid(c, E4M3_P, E4M3_EMIN)


def block_scale_pow2(amax):
    """The block scale for a block whose largest magnitude is amax (fp32):
    the smallest power of two s = 2^e with amax <= 448 * s, e >= -127 (the
    range of an E8M0 scale byte); s = 1 when amax = 0.  Written with an exact
    frexp split, amax = m * 2^E with m in [0.5, 1): 448 = 0.875 * 2^9, so
    e = E - 9 when m <= 0.875, else E - 8."""
    amax = np.asarray(amax, dtype=np.float32)
    out = np.ones(amax.shape, dtype=np.float32)
    nz = amax > 0
    m, E = np.frexp(amax[nz].astype(np.float64))
    e = np.maximum(np.where(m <= 0.875, E - 9, E - 8), -127)
    out[nz] = np.ldexp(1.0, e).astype(np.float32)
    return out


def block_scale_amax(amax):
    """The alternative block scale s = amax / 448 in fp32 (1 when amax = 0):
    the block's largest magnitude lands exactly on the largest e4m3 code.  Not
    used by the layer (its activation scales are powers of two, see
    block_scale_pow2); kept to measure what that choice costs in precision."""
    amax = np.asarray(amax, dtype=np.float32)
    with np.errstate(under="ignore"):
        s = (amax / np.float32(448.0)).astype(np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def quantize_fp8_blocks(v, block: int = FP8_BLOCK, rule: str = "pow2"):
    """Block-wise fp8 quantisation along the last axis.

    For each run of ``block`` consecutive elements (the last run may be
    shorter): amax = max |v| in fp32, s = block_scale_pow2(amax) (the
    smallest power of two with amax / s <= 448; 1 when amax = 0), code =
    e4m3(v / s) with the division done in fp32 (exact: s is a power of two),
    clamped to +-448 and rounded to nearest even.  A power-of-two scale is the
    E8M0 convention of the microscaling formats; the matrix cores apply such a
    scale themselves.

    Returns (codes, scales): codes are fp64 values on the e4m3 grid with the
    shape of ``v``; scales are fp32 with the last axis replaced by the number
    of blocks.  The represented value is codes * scales (per block).
    rule = 'amax448' takes s = block_scale_amax(amax) instead (the division
    is then an fp32 division that rounds).
    """
    if rule not in ("pow2", "amax448"):
        raise ValueError(f"unknown scale rule {rule!r}")
    scale_of = block_scale_pow2 if rule == "pow2" else block_scale_amax
    v32 = np.asarray(v, dtype=np.float32)
    n = v32.shape[-1]
    nb = -(-n // block)
    codes = np.empty(v32.shape, dtype=np.float64)
    scales = np.empty(v32.shape[:-1] + (nb,), dtype=np.float32)
    for b in range(nb):
        blk = v32[..., b * block:(b + 1) * block]
        amax = np.max(np.abs(blk), axis=-1)
        s = scale_of(amax)
        with np.errstate(over="ignore", under="ignore"):
            ratio = (blk / s[..., None]).astype(np.float32)   # fp32 division
        codes[..., b * block:(b + 1) * block] = to_e4m3_sat(ratio.astype(np.float64))
        scales[..., b] = s
    return codes, scales


def dequantize_fp8_blocks(codes, scales, block: int = FP8_BLOCK) -> np.ndarray:
    """codes * scale of the block each element belongs to, in fp64."""
    codes = np.asarray(codes, dtype=np.float64)
    n = codes.shape[-1]
    s = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=-1)[..., :n]
    return codes * s


def round_act(v, dtype: str, rule: str = "pow2"):
    """Round activations to the storage type named by ``dtype``.

    'f32' and 'bf16' return fp64 values on that grid; 'fp8' returns the
    (codes, scales) pair of :func:`quantize_fp8_blocks` (scale rule ``rule``)
    taken on the fp32 rounding of ``v``.
    """
    if dtype == "f32":
        return to_f32(v)
    if dtype == "bf16":
        return to_bf16(v)
    if dtype == "fp8":
        return quantize_fp8_blocks(to_f32(v), rule=rule)
    raise ValueError(f"unknown dtype {dtype!r}")
