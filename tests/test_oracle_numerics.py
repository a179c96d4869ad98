"""Pins of the oracle's rounding helpers against torch's CPU casts."""
import numpy as np
import pytest
import torch

from oracle import numerics as nx


def _all_bf16_values():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    with np.errstate(invalid="ignore"):
        v = bits.view(torch.bfloat16).float().numpy().astype(np.float64)
    return v[np.isfinite(v)]


def test_bf16_grid_is_fixed_point():
    v = _all_bf16_values()
    np.testing.assert_array_equal(nx.to_bf16(v), v)


def test_bf16_matches_torch_on_midpoints_and_random():
    v = _all_bf16_values()
    v = np.sort(v[v > 0])
    mids = (v[:-1] + v[1:]) / 2            # exact ties: fp64 holds them
    rng = np.random.default_rng(0)
    rnd = rng.normal(size=200_000) * np.exp(rng.uniform(-30, 30, size=200_000))
    for arr in (mids, -mids, rnd):
        f32 = arr.astype(np.float32)        # torch casts from fp32
        ok = f32.astype(np.float64) == arr  # compare only where fp32 is exact
        ref = torch.from_numpy(f32[ok]).to(torch.bfloat16).float().numpy()
        np.testing.assert_array_equal(nx.to_bf16(arr[ok]), ref)


def test_e4m3_all_codes_and_midpoints():
    codes = torch.arange(0, 256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    v = codes.float().numpy().astype(np.float64)
    v = v[np.isfinite(v)]
    np.testing.assert_array_equal(nx.to_e4m3_sat(v), v)
    pos = np.sort(np.unique(v[v > 0]))
    mids = (pos[:-1] + pos[1:]) / 2
    for arr in (mids, -mids, np.linspace(-448, 448, 100_001)):
        a32 = arr.astype(np.float32)          # torch casts from fp32
        ref = torch.from_numpy(a32).to(torch.float8_e4m3fn).float().numpy()
        np.testing.assert_array_equal(nx.to_e4m3_sat(a32.astype(np.float64)), ref)


def test_e4m3_saturates():
    np.testing.assert_array_equal(nx.to_e4m3_sat([1e9, -1e9, 465.0]), [448.0, -448.0, 448.0])


def test_fp8_block_quantiser_properties():
    rng = np.random.default_rng(1)
    v = rng.normal(size=(5, 2880)).astype(np.float32) * np.float32(3.0)
    v[2, 128:256] = 0.0                                   # an all-zero block
    codes, scales = nx.quantize_fp8_blocks(v)
    assert scales.shape == (5, 23) and scales.dtype == np.float32   # 22 full blocks + 64 tail
    assert scales[2, 1] == 1.0 and np.all(codes[2, 128:256] == 0)
    for b in range(23):
        blk = codes[:, b * 128:(b + 1) * 128]
        nz = np.abs(v[:, b * 128:(b + 1) * 128]).max(axis=1) > 0
        # the block's largest magnitude lands in the top binade of the codes
        # (amax / s is in (224, 448]; rounding can bring it down to 224)
        top = np.abs(blk[nz]).max(axis=1)
        assert np.all((top >= 224.0) & (top <= 448.0))
    # scales are powers of two
    m, _ = np.frexp(scales.astype(np.float64))
    assert np.all(m == 0.5)
    deq = nx.dequantize_fp8_blocks(codes, scales)
    amax = np.repeat(np.abs(v.reshape(5, -1)).max(axis=1, keepdims=True), 2880, axis=1)
    # error <= half an e4m3 step of the top binade: 16 * s, and s < 2 * amax / 448
    assert np.all(np.abs(deq - v) <= amax / 448 * 32 * 1.0001)


def test_fp8_scale_rule_by_hand():
    """amax 3.5: 3.5/448 = 2^-7 exactly, so s = 2^-7 and 3.5 -> 448, -1 -> -128.
    amax 7.5: 7.5/448 lies in (2^-6, 2^-5], so s = 2^-5 and 7.5 -> 240.
    amax 448 -> s = 1; amax 449 -> s = 2; amax 2^-140 -> s = 2^-127 (E8M0 floor)."""
    v = np.zeros((1, 136), np.float32)
    v[0, 0] = 3.5
    v[0, 5] = -1.0
    v[0, 130] = 7.5
    codes, scales = nx.quantize_fp8_blocks(v)
    assert scales[0, 0] == np.float32(2.0 ** -7)
    assert scales[0, 1] == np.float32(2.0 ** -5)
    assert codes[0, 0] == 448.0 and codes[0, 5] == -128.0
    assert codes[0, 130] == 240.0
    assert list(nx.block_scale_pow2([448.0, 449.0, 0.0, 2.0 ** -140, 1.0])) == \
        [1.0, 2.0, 1.0, np.float32(2.0 ** -127), np.float32(2.0 ** -8)]


def test_round_to_grid_subnormals():
    # bf16 smallest subnormal is 2^-133; half of it ties to even (zero)
    assert nx.to_bf16(2.0**-134) == 0.0
    assert nx.to_bf16(3 * 2.0**-134) == 2.0**-132
    # e4m3 smallest subnormal is 2^-9
    assert nx.to_e4m3_sat(2.0**-10) == 0.0
    assert nx.to_e4m3_sat(3 * 2.0**-10) == 2.0**-8


def test_block_scale_amax_rule_by_hand():
    """The alternative scale rule s = amax / 448 (fp32; 1 for an all-zero
    block): 448 -> 1, 896 -> 2, 0 -> 1, 1 -> fp32(1/448); quantising with it
    puts each block's largest magnitude on the top code 448 (the division
    rounds in fp32, so within one code of it) and the pow2 rule's scale is
    never smaller."""
    s = nx.block_scale_amax([448.0, 896.0, 0.0, 1.0])
    assert s.dtype == np.float32
    assert list(s[:3]) == [1.0, 2.0, 1.0]
    assert s[3] == np.float32(1.0) / np.float32(448.0)
    rng = np.random.default_rng(3)
    v = rng.standard_normal((5, 300)) * np.exp(rng.standard_normal((5, 1)))
    codes, sc = nx.quantize_fp8_blocks(v, rule="amax448")
    for b in range(3):
        top = np.max(np.abs(codes[:, b * 128:(b + 1) * 128]), axis=1)
        assert np.all((top == 448.0) | (top == 416.0)), top
    _, sp = nx.quantize_fp8_blocks(v)
    assert np.all(sp >= sc)
    with pytest.raises(ValueError):
        nx.quantize_fp8_blocks(v, rule="other")
