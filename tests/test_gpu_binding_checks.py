"""The binding refuses caller-provided tensors too small for what the kernels
index, with ValueError before any library call (the C ABI sees only
pointers: an undersized output would be written out of bounds)."""
import pytest
import torch

from harness import has_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _t(shape, dtype=torch.int32):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_route_and_layout_outputs():
    import combine_grouped_gemm_amd as m
    logits = torch.randn(10, 16, device="cuda")
    with pytest.raises(ValueError, match="topk_ids"):
        m.moe_route(logits, 2, topk_ids=_t((10, 1)))
    with pytest.raises(ValueError, match="topk_w"):
        m.moe_route(logits, 2, topk_w=_t((9, 2), torch.float32))
    ids = _t((10, 2))
    for kw, name in ((dict(counts=_t(15)), "counts"), (dict(offsets=_t(8)), "offsets"),
                     (dict(row_of=_t((10, 1))), "row_of"), (dict(src_of=_t(19)), "src_of")):
        with pytest.raises(ValueError, match=name):
            m.moe_layout(ids, 16, 4, 12, 20, **kw)
        with pytest.raises(ValueError, match=name):
            m.moe_layout_noalloc(ids, 16, 4, 12, 20, **kw)
    with pytest.raises(ValueError, match="src_of"):
        m.moe_layout_masked(ids, 16, 4, 12, 5, src_of=_t(39))
    with pytest.raises(ValueError, match="m needs"):
        m.moe_layout_masked(ids, 16, 4, 12, 5, m=_t(7))
    torch.cuda.synchronize()


def test_dispatch_combine_ffn_outputs():
    import combine_grouped_gemm_amd as m
    H, I, E, K, T = 128, 64, 4, 2, 6
    x = torch.randn(T, H, device="cuda").to(torch.bfloat16)
    row_of = _t((T, K))
    with pytest.raises(ValueError, match="xd"):
        m.moe_dispatch(x, row_of, T * K, xd=_t((T * K - 1, H), torch.bfloat16))
    with pytest.raises(ValueError, match="xd_scales"):
        m.moe_dispatch(x, row_of, T * K, "fp8", xd=_t((T * K, H), torch.float8_e4m3fn),
                       xd_scales=_t((T * K - 1, 1), torch.float32))
    with pytest.raises(ValueError, match="row_of"):
        m.moe_dispatch(x, _t((T - 1, K)), T * K)
    xd = _t((T * K, H), torch.bfloat16)
    offsets = _t(E + 1)
    wg = _t((E, I, H), torch.bfloat16)
    wd = _t((E, H, I), torch.bfloat16)
    with pytest.raises(ValueError, match="w_up"):
        m.moe_ffn_gate_up(xd, None, offsets, wg, _t((E, I - 16, H), torch.bfloat16))
    with pytest.raises(ValueError, match="h needs"):
        m.moe_ffn_gate_up(xd, None, offsets, wg, wg, h=_t((T * K - 1, I), torch.bfloat16))
    with pytest.raises(ValueError, match="offsets"):
        m.moe_ffn_gate_up(xd, None, _t(E), wg, wg)
    h = _t((T * K, I), torch.bfloat16)
    with pytest.raises(ValueError, match="y needs"):
        m.moe_ffn_down(h, None, offsets, wd, y=_t((T * K, H - 8), torch.bfloat16))
    with pytest.raises(ValueError, match="w_down"):
        m.moe_grouped_ffn(xd, None, offsets, wg, wg, _t((E, H, I + 16), torch.bfloat16))
    y = _t((T * K, H), torch.bfloat16)
    with pytest.raises(ValueError, match="out needs"):
        m.moe_combine(y, row_of, _t((T, K), torch.float32), out=_t((T - 1, H), torch.bfloat16))
    with pytest.raises(ValueError, match="topk_w"):
        m.moe_combine(y, row_of, _t((T, K - 1), torch.float32))
    torch.cuda.synchronize()
