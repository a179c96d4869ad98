"""The allocation-free layout entry point (moe_layout_noalloc), through the
C ABI, against moe_layout with a caller workspace: bit-identical counts,
offsets, row_of and src_of on two calls in a row, the second with a smaller
batch (the library's scratch keeps the first call's contents), and again
after a batch that needs no workspace at all."""
import numpy as np
import pytest
import torch

from harness import has_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _ids(B, K, E, seed):
    g = torch.Generator().manual_seed(seed)
    lg = torch.randn(B, E, generator=g)
    return torch.topk(lg, K, dim=1).indices.to(torch.int32).contiguous().cuda()


def _same(a, b):
    for k in ("counts", "offsets", "row_of", "src_of"):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("shapes", [
    # (B, K, E, e_begin, e_end): prefill-sized, then smaller with other experts,
    # then one that takes the single-workgroup path, then a mid-sized one
    [(8192, 8, 256, 0, 256), (1000, 8, 64, 16, 48), (300, 8, 32, 0, 32), (2600, 4, 128, 32, 96)],
])
def test_noalloc_layout_matches_workspace_layout(shapes):
    import combine_grouped_gemm_amd as m
    for i, (B, K, E, eb, ee) in enumerate(shapes):
        print(f"[no-alloc] call {i}: B={B} K={K} E={E} local [{eb}, {ee})", flush=True)
        assert m.moe_layout_workspace_bytes(B, K, E) <= m.LAYOUT_NOALLOC_SCRATCH_BYTES
        ids = _ids(B, K, E, seed=100 + i)
        cap = B * K
        ref = m.moe_layout(ids, E, eb, ee, cap)
        got = m.moe_layout_noalloc(ids, E, eb, ee, cap)
        torch.cuda.synchronize()
        _same(got, ref)
        # sanity of the reference itself: a permutation onto the local rows
        R = int(ref["offsets"][-1])
        src = ref["src_of"][:R].cpu().numpy()
        assert np.array_equal(np.sort(src), np.sort(np.nonzero((ids.cpu().numpy().reshape(-1) >= eb)
                                                               & (ids.cpu().numpy().reshape(-1) < ee))[0]))


def test_noalloc_layout_allocates_nothing_with_given_outputs():
    """With every output given, a call adds nothing to torch's device
    allocations (the library allocates nothing itself either: its scratch is
    a static device array)."""
    import combine_grouped_gemm_amd as m
    B, K, E = 4000, 8, 256
    ids = _ids(B, K, E, seed=7)
    outs = dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
                offsets=torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                row_of=torch.empty((B, K), dtype=torch.int32, device="cuda"),
                src_of=torch.empty(B * K, dtype=torch.int32, device="cuda"))
    m.moe_layout_noalloc(ids, E, 0, E, B * K, **outs)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for _ in range(3):
        m.moe_layout_noalloc(ids, E, 0, E, B * K, **outs)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    ref = m.moe_layout(ids, E, 0, E, B * K)
    torch.cuda.synchronize()
    _same(outs, ref)
