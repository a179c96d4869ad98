"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import combine_grouped_gemm_amd as m

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moeep.h")


def declared():
    text = open(HDR).read()
    return re.findall(r"^\s*(?:moe_status_t|size_t|int|const char\*)\s+(moe_\w+)\(", text, re.M)


def test_exports_every_declared_symbol():
    L = m.lib()
    names = declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = m.lib()
    assert L.moe_status_string(0) == b"MOE_OK"
    assert L.moe_status_string(3) == b"MOE_ERR_HIP"
    assert b"gfx950" in L.moe_version()


BAD_ROUTE = [((None, 4, 0, 1), "E must be"), ((None, 4, 8, 9), "K must be"),
             ((None, -1, 8, 2), "B must be"), ((None, 4, 2000, 2), "E must be"),
             ((None, 4, 8, 2), "null pointer")]


@pytest.mark.parametrize("args,msg", BAD_ROUTE)
def test_route_rejects(args, msg):
    L = m.lib()
    assert L.moe_route(*args, None, None, None) == m.MOE_ERR_INVALID_ARG
    assert msg in L.moe_last_error().decode()


def test_route_empty_batch_is_noop():
    assert m.lib().moe_route(None, 0, 8, 2, None, None, None) == m.MOE_OK


def test_layout_rejects():
    L = m.lib()
    p = ctypes.c_void_p(256)       # never dereferenced: every case fails its host check first
    assert L.moe_layout(p, 4, 2, 8, 3, 3, p, p, p, p, 8, p, 1 << 20, None) == m.MOE_ERR_INVALID_ARG
    assert "e_begin" in L.moe_last_error().decode()
    assert L.moe_layout(p, 4, 2, 8, 0, 8, p, p, p, p, 8, ctypes.c_void_p(257), 1 << 20, None) == 1
    assert "256-byte" in L.moe_last_error().decode()
    assert L.moe_layout(p, 4, 2, 8, 0, 8, p, p, p, p, 8, p, 4, None) == m.MOE_ERR_INVALID_ARG
    assert "workspace too small" in L.moe_last_error().decode()
    assert L.moe_layout_workspace_bytes(8192, 8, 256) % 256 == 0


def test_dispatch_rejects():
    L = m.lib()
    p = ctypes.c_void_p(4096)
    ptrs = (ctypes.c_void_p * 1)(4096)
    rows = (ctypes.c_int32 * 1)(4)
    P = lambda a: ctypes.cast(a, ctypes.c_void_p)
    assert L.moe_dispatch(P(ptrs), P(rows), 0, 1, 128, p, 2, p, 1, None, 8, None) == 1
    assert L.moe_dispatch(P(ptrs), P(rows), 1, 1, 100, p, 2, p, 1, None, 8, None) == 1   # H % 8
    assert L.moe_dispatch(P(ptrs), P(rows), 1, 1, 0, p, 2, p, 1, None, 8, None) == 1     # H >= 8
    # fp8 rows need H % 16 (the fp8 GEMMs move 16-byte pieces)
    assert L.moe_dispatch(P(ptrs), P(rows), 1, 1, 200, p, 2, p, 2, p, 8, None) == 1
    assert "multiple of 16" in L.moe_last_error().decode()
    assert L.moe_dispatch(P(ptrs), P(rows), 1, 0, 128, p, 2, p, 2, None, 8, None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_dispatch(P(ptrs), P(rows), 1, 1, 128, p, 2, p, 2, None, 8, None) == 1   # fp8 needs scales
    ptrs[0] = 4097
    assert L.moe_dispatch(P(ptrs), P(rows), 1, 1, 128, p, 2, p, 1, None, 8, None) == 1   # misaligned
    assert "aligned" in L.moe_last_error().decode()


def test_ffn_rejects():
    L = m.lib()
    p = ctypes.c_void_p(4096)
    # bf16 activations with fp8 weights: unsupported
    assert L.moe_ffn_gate_up(p, None, p, 8, 64, 128, 128, 1, p, p, None, None, 2, p, None, 0, None) == 2
    # I not a multiple of 8
    assert L.moe_ffn_gate_up(p, None, p, 8, 64, 128, 100, 1, p, p, None, None, 1, p, None, 0, None) == 1
    assert "multiples of 8" in L.moe_last_error().decode()
    # fp8: H and I multiples of 16
    assert L.moe_ffn_gate_up(p, p, p, 8, 64, 200, 128, 2, p, p, p, p, 2, p, p, 0, None) == 1
    assert "multiples of 16" in L.moe_last_error().decode()
    # fp8 without scales
    assert L.moe_ffn_gate_up(p, None, p, 8, 64, 128, 128, 2, p, p, None, None, 2, p, None, 0, None) == 1
    # fp8 activations need a bf16 y
    assert L.moe_ffn_down(p, p, p, 8, 64, 128, 128, 2, p, p, 2, p, 2, 0, None) == 2
    # power-of-two-scale fp8 is a weight dtype only: not with bf16 activations, not as activations
    assert L.moe_ffn_gate_up(p, None, p, 8, 64, 128, 128, 1, p, p, None, None, 3, p, None, 0, None) == 2
    assert L.moe_ffn_gate_up(p, p, p, 8, 64, 128, 128, 3, p, p, p, p, 3, p, p, 0, None) == 2
    assert L.moe_ffn_down(p, p, p, 8, 64, 128, 128, 2, p, None, 3, p, 1, 0, None) == 1   # scales needed
    assert L.moe_dispatch(ctypes.cast((ctypes.c_void_p * 1)(4096), ctypes.POINTER(ctypes.c_void_p)),
                          (ctypes.c_int32 * 1)(4), 1, 1, 128, p, 2, p, 3, p, 8, None) == 2
    # workspace too small
    assert L.moe_grouped_ffn(p, None, p, 8, 64, 128, 128, 1, p, p, p, None, None, None, 1, p, 1,
                             p, 16, 0, None) == 1
    assert L.moe_ffn_workspace_bytes(64, 128, 2) >= 64 * 128 + 64 * 4


def test_combine_rejects():
    L = m.lib()
    p = ctypes.c_void_p(4096)
    assert L.moe_combine(p, 2, 8, p, p, 4, 2, 128, p, 1, None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_combine(p, 1, 8, p, p, 4, 2, 124, p, 1, None) == m.MOE_ERR_INVALID_ARG   # H % 8
    assert L.moe_combine(p, 1, 8, None, p, 4, 2, 128, p, 1, None) == m.MOE_ERR_INVALID_ARG


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        m.moe_route(torch.zeros(4, 8), 2)


def test_masked_entry_points_reject():
    L = m.lib()
    p = ctypes.c_void_p(4096)
    # layout: cap_per_expert must be >= 1, E_local * cap_per_expert must fit in int32
    assert L.moe_layout_masked(p, 4, 2, 8, 0, 8, p, p, p, p, 0, p, 1 << 20, None) == m.MOE_ERR_INVALID_ARG
    assert "cap_per_expert" in L.moe_last_error().decode()
    assert L.moe_layout_masked(p, 4, 2, 1024, 0, 1024, p, p, p, p, 1 << 22, p, 1 << 20, None) == 1
    assert "fit in int32" in L.moe_last_error().decode()
    assert L.moe_layout_masked(p, 4, 2, 8, 0, 8, p, None, p, p, 4, p, 1 << 20, None) == 1
    assert "null" in L.moe_last_error().decode()
    # FFN: m must be given; the shared checks still apply
    assert L.moe_ffn_gate_up_masked(p, None, None, 4, 16, 128, 128, 1, p, p, None, None, 1, p,
                                    None, 0, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_ffn_down_masked(p, None, p, 4, 0, 128, 128, 1, p, None, 1, p, 1, 0, None) == 1
    assert "cap_per_expert" in L.moe_last_error().decode()
    assert L.moe_grouped_ffn_masked(p, None, p, 4, 16, 100, 128, 1, p, p, p, None, None, None, 1,
                                    p, 1, p, 1 << 30, 0, None) == m.MOE_ERR_INVALID_ARG
    assert "multiples of 8" in L.moe_last_error().decode()


def test_eplb_place_matches_oracle_and_rejects():
    """The library's host placement is the oracle's reading, id for id."""
    import numpy as np
    from oracle import eplb
    rng = np.random.default_rng(7)
    for E, G in [(8, 2), (16, 4), (256, 8), (12, 3), (64, 64), (40, 1), (1024, 8)]:
        for _ in range(5):
            load = rng.integers(0, 2000, size=E) * rng.integers(0, 2, size=E)   # with zero loads and ties
            got = m.moe_eplb_place(load, G).numpy()
            np.testing.assert_array_equal(got, eplb.balanced_placement(load, G))
    L = m.lib()
    buf = (ctypes.c_int64 * 10)(*range(10))
    out = (ctypes.c_int32 * 10)()
    P = lambda a: ctypes.cast(a, ctypes.c_void_p)
    assert L.moe_eplb_place(P(buf), 10, 3, P(out)) == m.MOE_ERR_INVALID_ARG
    assert "divide" in L.moe_last_error().decode()
    buf[4] = -1
    assert L.moe_eplb_place(P(buf), 10, 2, P(out)) == m.MOE_ERR_INVALID_ARG
    assert L.moe_route_mapped(None, 4, 8, 2, None, None, None, None) == m.MOE_ERR_INVALID_ARG


def test_route_shared_rejects():
    L = m.lib()
    p = ctypes.c_void_p(4096)
    assert L.moe_route_shared(p, 4, 1000, 8, 30, p, p, None) == m.MOE_ERR_INVALID_ARG
    assert "n_shared" in L.moe_last_error().decode()
    assert L.moe_route_shared(p, 4, 16, 2, -1, p, p, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_route_shared(None, 0, 16, 2, 1, None, None, None) == m.MOE_OK


def test_layout_noalloc_rejects_before_any_hip_call():
    """The allocation-free layout checks everything on the host first: a batch
    whose chunk histograms exceed the library's scratch is refused with a
    message naming the limit, before the scratch is looked up."""
    L = m.lib()
    p = ctypes.c_void_p(256)
    limit = m.LAYOUT_NOALLOC_SCRATCH_BYTES
    # E = 1024, B*K = 2^20 slots: 4096 chunks x 1024 experts x 4 bytes = 16 MiB
    assert L.moe_layout_workspace_bytes(1 << 17, 8, 1024) > limit
    assert L.moe_layout_noalloc(p, 1 << 17, 8, 1024, 0, 1024, p, p, p, p, 1 << 20, None) == \
        m.MOE_ERR_INVALID_ARG
    msg = L.moe_last_error().decode()
    assert "moe_layout_noalloc" in msg and str(limit) in msg
    assert L.moe_layout_noalloc(p, 4, 2, 8, 5, 5, p, p, p, p, 8, None) == m.MOE_ERR_INVALID_ARG
    assert "e_begin" in L.moe_last_error().decode()
    assert L.moe_layout_noalloc(p, 4, 2, 8, 0, 8, None, p, p, p, 8, None) == m.MOE_ERR_INVALID_ARG
    # the prefill batch (T = 8192, K = 8, E = 256) fits
    assert L.moe_layout_workspace_bytes(8192, 8, 256) <= limit


# (cols, dtype code, packed pitch in elements): whole 128-byte lines, one more
# line when the row is a multiple of 4 KiB
PITCHES = [(2048, m.MOE_BF16, 2112), (7168, m.MOE_BF16, 7168), (2880, m.MOE_FP8_E4M3, 2944),
           (2880, m.MOE_FP8_E4M3_PO2, 2944), (4096, m.MOE_FP8_E4M3, 4224), (128, m.MOE_F32, 128),
           (1024, m.MOE_F32, 1056), (256, m.MOE_F32, 256), (8, m.MOE_BF16, 64),
           (2048, m.MOE_BF16 | m.MOE_W_PACKED, 2112)]


@pytest.mark.parametrize("cols,dt,ld", PITCHES)
def test_weight_ld(cols, dt, ld):
    L = m.lib()
    assert L.moe_weight_ld(cols, dt) == ld
    esz = {m.MOE_F32: 4, m.MOE_BF16: 2}.get(dt & ~m.MOE_W_PACKED, 1)
    assert ld * esz % 128 == 0 and ld >= cols and (ld * esz) % 4096 != 0
    assert L.moe_packed_weight_bytes(3, 5, cols, dt) == 3 * 5 * ld * esz


def test_weight_ld_rejects():
    L = m.lib()
    assert L.moe_weight_ld(0, m.MOE_BF16) == -1
    assert L.moe_weight_ld(64, 7) == -1
    assert L.moe_packed_weight_bytes(2, 2, 64, 7) == 0


def test_pack_weights_rejects_before_any_hip_call():
    L = m.lib()
    p, q = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 30)    # never dereferenced
    assert L.moe_pack_weights(p, 2, 4, 64, 7, q, None) == m.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_weights(p, 2, 4, 60, m.MOE_BF16, q, None) == m.MOE_ERR_INVALID_ARG
    assert "multiple of 8" in L.moe_last_error().decode()
    assert L.moe_pack_weights(None, 2, 4, 64, m.MOE_BF16, q, None) == m.MOE_ERR_INVALID_ARG
    assert L.moe_pack_weights(ctypes.c_void_p((1 << 20) + 8), 2, 4, 64, m.MOE_BF16, q, None) == 1
    assert "16-byte" in L.moe_last_error().decode()
    # 8 rows of 128 bytes packed to 8 rows of 128: [p, p + 1 KiB) and [p + 512, ...) overlap
    assert L.moe_pack_weights(p, 2, 4, 64, m.MOE_BF16, ctypes.c_void_p((1 << 20) + 512), None) == 1
    assert "overlap" in L.moe_last_error().decode()
    assert L.moe_pack_weights(None, 0, 4, 64, m.MOE_BF16, None, None) == m.MOE_OK
