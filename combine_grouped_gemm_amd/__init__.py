"""Python binding of libmoeep: the single-GPU expert-parallel MoE layer path
(route -> layout -> dispatch -> grouped SwiGLU FFN -> combine) on MI355X.

Each function here has the name of the C entry point it marshals (see
include/moeep.h for the full contract).  Tensors are torch device tensors
used only as memory; the binding checks shapes and dtypes, allocates outputs
the caller did not provide, passes ``data_ptr()`` and the current HIP stream,
and raises :class:`MoeError` with the library's message on a non-OK status.
All compute happens in the HIP kernels of ``libmoeep.so``; there is no other
code path.  Build the library with ``python -m combine_grouped_gemm_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["MoeError", "lib", "library_path", "moe_version", "moe_route",
           "moe_layout_workspace_bytes", "moe_layout", "moe_layout_noalloc", "moe_dispatch",
           "moe_ffn_workspace_bytes", "moe_ffn_gate_up", "moe_ffn_down",
           "moe_grouped_ffn", "moe_combine", "moe_layout_masked", "moe_ffn_gate_up_masked",
           "moe_ffn_down_masked", "moe_grouped_ffn_masked", "moe_route_mapped", "moe_eplb_place", "moe_route_shared",
           "moe_weight_ld", "moe_packed_weight_bytes", "moe_pack_weights",
           "MOE_F32", "MOE_BF16", "MOE_FP8_E4M3", "MOE_FP8_E4M3_PO2", "MOE_W_PACKED",
           "MoELayer"]

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 0, 1, 2, 3
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_FP8_E4M3_PO2 = 0, 1, 2, 3
MOE_W_PACKED = 0x100
FP8_BLOCK = 128
MAX_SEGMENTS = 64

_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.float8_e4m3fn: MOE_FP8_E4M3}
_TORCH = {v: k for k, v in _DT.items()}
_NAMES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoeep.so")
_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


def _status_name(s):
    return {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
            3: "MOE_ERR_HIP"}.get(s, f"status {s}")


def lib() -> ctypes.CDLL:
    """The loaded libmoeep.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"libmoeep.so is missing at {library_path}; build it with "
                           "'python -m combine_grouped_gemm_amd.build'")
    L = ctypes.CDLL(library_path)
    P, I, Z, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int
    sig = {
        "moe_status_string": ([I], ctypes.c_char_p),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_version": ([], ctypes.c_char_p),
        "moe_route": ([P, I, I, I, P, P, P], S),
        "moe_layout_workspace_bytes": ([I, I, I], Z),
        "moe_layout": ([P, I, I, I, I, I, P, P, P, P, I, P, Z, P], S),
        "moe_layout_noalloc": ([P, I, I, I, I, I, P, P, P, P, I, P], S),
        "moe_dispatch": ([P, P, I, I, I, P, I, P, I, P, I, P], S),
        "moe_ffn_workspace_bytes": ([I, I, I], Z),
        "moe_ffn_gate_up": ([P, P, P, I, I, I, I, I, P, P, P, P, I, P, P, I, P], S),
        "moe_ffn_down": ([P, P, P, I, I, I, I, I, P, P, I, P, I, I, P], S),
        "moe_grouped_ffn": ([P, P, P, I, I, I, I, I, P, P, P, P, P, P, I, P, I, P, Z, I, P], S),
        "moe_combine": ([P, I, I, P, P, I, I, I, P, I, P], S),
        "moe_layout_masked": ([P, I, I, I, I, I, P, P, P, P, I, P, Z, P], S),
        "moe_route_mapped": ([P, I, I, I, P, P, P, P], S),
        "moe_eplb_place": ([P, I, I, P], S),
        "moe_route_shared": ([P, I, I, I, I, P, P, P], S),
        "moe_weight_ld": ([I, I], I),
        "moe_packed_weight_bytes": ([I, I, I, I], Z),
        "moe_pack_weights": ([P, I, I, I, I, P, P], S),
    }
    # the masked FFN calls take (m, E_local, cap_per_expert) where the others take
    # (offsets, E_local, cap_rows): same argument types
    for name in ("moe_ffn_gate_up", "moe_ffn_down", "moe_grouped_ffn"):
        sig[name + "_masked"] = sig[name]
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes, f.restype = args, res
    _lib = L
    return L


def _check(status: int):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {t.dim()})")
    return t


def _need(t, name, numel=None, shape=None):
    """Caller-provided tensors must cover what the kernels index: the C ABI
    cannot see sizes, so an undersized tensor would be written out of bounds
    on the device.  Raises ValueError before any library call."""
    if t is None:
        return
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements (got {t.numel()})")


def _dtype_code(d):
    if isinstance(d, str):
        return _NAMES[d]
    if isinstance(d, torch.dtype):
        return _DT[d]
    return int(d)


def moe_version() -> str:
    return lib().moe_version().decode()


# ----------------------------------------------------------------------------
def moe_route(logits, K: int, topk_ids=None, topk_w=None, stream=None):
    """Top-K expert ids (B, K) int32 and renormalised softmax gates (B, K) fp32."""
    _dev(logits, "logits", torch.float32, 2)
    B, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((B, K), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((B, K), dtype=torch.float32, device=logits.device)
    _dev(topk_ids, "topk_ids", torch.int32)
    _dev(topk_w, "topk_w", torch.float32)
    _need(topk_ids, "topk_ids", shape=(B, K))
    _need(topk_w, "topk_w", shape=(B, K))
    _check(lib().moe_route(_ptr(logits), B, E, K, _ptr(topk_ids), _ptr(topk_w), _stream(stream)))
    return topk_ids, topk_w


def moe_route_mapped(logits, K: int, phys_of_logical, topk_ids=None, topk_w=None, stream=None):
    """moe_route with the chosen expert ids written through a placement map
    (phys_of_logical: (E,) int32 device tensor)."""
    _dev(logits, "logits", torch.float32, 2)
    _dev(phys_of_logical, "phys_of_logical", torch.int32, 1)
    B, E = logits.shape
    if phys_of_logical.numel() != E:
        raise ValueError("phys_of_logical needs E entries")
    if topk_ids is None:
        topk_ids = torch.empty((B, K), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((B, K), dtype=torch.float32, device=logits.device)
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    _dev(topk_w, "topk_w", torch.float32, 2)
    _need(topk_ids, "topk_ids", shape=(B, K))
    _need(topk_w, "topk_w", shape=(B, K))
    _check(lib().moe_route_mapped(_ptr(logits), B, E, K, _ptr(phys_of_logical), _ptr(topk_ids),
                                  _ptr(topk_w), _stream(stream)))
    return topk_ids, topk_w


def moe_route_shared(logits, K: int, n_shared: int, topk_ids=None, topk_w=None, stream=None):
    """moe_route plus n_shared always-on experts: ids / gates (B, K + n_shared),
    the last n_shared columns E, E+1, ... with gate 1."""
    _dev(logits, "logits", torch.float32, 2)
    B, E = logits.shape
    Kt = K + n_shared
    if topk_ids is None:
        topk_ids = torch.empty((B, Kt), dtype=torch.int32, device=logits.device)
    if topk_w is None:
        topk_w = torch.empty((B, Kt), dtype=torch.float32, device=logits.device)
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    _dev(topk_w, "topk_w", torch.float32, 2)
    if topk_ids.shape != (B, Kt) or topk_w.shape != (B, Kt):
        raise ValueError(f"outputs must be ({B}, {Kt})")
    _check(lib().moe_route_shared(_ptr(logits), B, E, K, int(n_shared), _ptr(topk_ids), _ptr(topk_w),
                                  _stream(stream)))
    return topk_ids, topk_w


def moe_eplb_place(load, n_groups: int):
    """Host expert placement: load (E,) activation counts (any integer
    array-like) -> phys_of_logical (E,) int32 CPU tensor."""
    load = torch.as_tensor(load).to(torch.int64).contiguous().cpu()
    if load.dim() != 1:
        raise ValueError("load must be 1-D")
    phys = torch.empty(load.numel(), dtype=torch.int32)
    _check(lib().moe_eplb_place(load.data_ptr(), load.numel(), int(n_groups), phys.data_ptr()))
    return phys


def moe_layout_workspace_bytes(B: int, K: int, E: int) -> int:
    return int(lib().moe_layout_workspace_bytes(B, K, E))


def _check_layout_outputs(B, K, E, E_loc, cap_rows, counts, offsets, row_of, src_of):
    _need(counts, "counts", numel=E)
    _need(offsets, "offsets", numel=max(E_loc, 0) + 1)
    _need(row_of, "row_of", numel=B * K)
    _need(src_of, "src_of", numel=cap_rows)


def moe_layout(topk_ids, E: int, e_begin: int, e_end: int, cap_rows: int, counts=None,
               offsets=None, row_of=None, src_of=None, ws=None, stream=None) -> dict:
    """counts (E), offsets (E_loc+1), row_of (B, K), src_of (cap_rows), all int32."""
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    B, K = topk_ids.shape
    dev = topk_ids.device
    E_loc = e_end - e_begin
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(max(E_loc, 0) + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    row_of = torch.empty((B, K), dtype=torch.int32, device=dev) if row_of is None else row_of
    src_of = torch.empty(max(cap_rows, 1), dtype=torch.int32, device=dev) if src_of is None else src_of
    need = moe_layout_workspace_bytes(B, K, E)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    for n, t in (("counts", counts), ("offsets", offsets), ("row_of", row_of), ("src_of", src_of)):
        _dev(t, n, torch.int32)
    _check_layout_outputs(B, K, E, E_loc, cap_rows, counts, offsets, row_of, src_of)
    _dev(ws, "ws")
    _check(lib().moe_layout(_ptr(topk_ids), B, K, E, e_begin, e_end, _ptr(counts), _ptr(offsets),
                            _ptr(row_of), _ptr(src_of), cap_rows, _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream)))
    return {"counts": counts, "offsets": offsets, "row_of": row_of, "src_of": src_of}


LAYOUT_NOALLOC_SCRATCH_BYTES = 4 << 20


def moe_layout_noalloc(topk_ids, E: int, e_begin: int, e_end: int, cap_rows: int, counts=None,
                       offsets=None, row_of=None, src_of=None, stream=None) -> dict:
    """moe_layout without a workspace argument: the library's own per-GPU
    scratch (LAYOUT_NOALLOC_SCRATCH_BYTES) holds the chunk histograms, and
    the call allocates nothing on the device when every output is given.
    Batches needing more workspace than that raise MoeError; calls that
    overlap on one GPU race on the shared scratch."""
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    B, K = topk_ids.shape
    dev = topk_ids.device
    E_loc = e_end - e_begin
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(max(E_loc, 0) + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    row_of = torch.empty((B, K), dtype=torch.int32, device=dev) if row_of is None else row_of
    src_of = torch.empty(max(cap_rows, 1), dtype=torch.int32, device=dev) if src_of is None else src_of
    for n, t in (("counts", counts), ("offsets", offsets), ("row_of", row_of), ("src_of", src_of)):
        _dev(t, n, torch.int32)
    _check_layout_outputs(B, K, E, E_loc, cap_rows, counts, offsets, row_of, src_of)
    _check(lib().moe_layout_noalloc(_ptr(topk_ids), B, K, E, e_begin, e_end, _ptr(counts), _ptr(offsets),
                                    _ptr(row_of), _ptr(src_of), cap_rows, _stream(stream)))
    return {"counts": counts, "offsets": offsets, "row_of": row_of, "src_of": src_of}


def moe_layout_masked(topk_ids, E: int, e_begin: int, e_end: int, cap_per_expert: int, counts=None,
                      m=None, row_of=None, src_of=None, ws=None, stream=None) -> dict:
    """Fixed-capacity layout: counts (E), m (E_loc), row_of (B, K),
    src_of (E_loc * cap_per_expert), all int32."""
    _dev(topk_ids, "topk_ids", torch.int32, 2)
    B, K = topk_ids.shape
    dev = topk_ids.device
    E_loc = e_end - e_begin
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    m = torch.empty(max(E_loc, 1), dtype=torch.int32, device=dev) if m is None else m
    row_of = torch.empty((B, K), dtype=torch.int32, device=dev) if row_of is None else row_of
    if src_of is None:
        src_of = torch.empty(max(E_loc * cap_per_expert, 1), dtype=torch.int32, device=dev)
    need = moe_layout_workspace_bytes(B, K, E)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    for n, t in (("counts", counts), ("m", m), ("row_of", row_of), ("src_of", src_of)):
        _dev(t, n, torch.int32)
    _need(counts, "counts", numel=E)
    _need(m, "m", numel=max(E_loc, 0))
    _need(row_of, "row_of", numel=B * K)
    _need(src_of, "src_of", numel=max(E_loc, 0) * cap_per_expert)
    _dev(ws, "ws")
    _check(lib().moe_layout_masked(_ptr(topk_ids), B, K, E, e_begin, e_end, _ptr(counts), _ptr(m),
                                   _ptr(row_of), _ptr(src_of), cap_per_expert, _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)))
    return {"counts": counts, "m": m, "row_of": row_of, "src_of": src_of}


def moe_dispatch(seg_x, row_of, cap_rows: int, xd_dtype=None, xd=None, xd_scales=None,
                 stream=None):
    """Scatter the token rows of the segments into xd (cap_rows, H); fp8
    storage also fills xd_scales (cap_rows, ceil(H/128))."""
    if isinstance(seg_x, torch.Tensor):
        seg_x = [seg_x]
    seg_x = list(seg_x)
    if not 1 <= len(seg_x) <= MAX_SEGMENTS:
        raise ValueError(f"need 1..{MAX_SEGMENTS} segments")
    x_dt = seg_x[0].dtype
    H = seg_x[0].shape[1]
    for i, s in enumerate(seg_x):
        _dev(s, f"seg_x[{i}]", x_dt, 2)
        if s.shape[1] != H:
            raise ValueError("all segments need the same H")
    _dev(row_of, "row_of", torch.int32, 2)
    K = row_of.shape[1]
    dev = row_of.device
    xd_code = _DT[x_dt] if xd_dtype is None else _dtype_code(xd_dtype)
    if xd is None:
        xd = torch.empty((max(cap_rows, 1), H), dtype=_TORCH[xd_code], device=dev)
    if xd_code == MOE_FP8_E4M3 and xd_scales is None:
        xd_scales = torch.empty((max(cap_rows, 1), -(-H // FP8_BLOCK)), dtype=torch.float32, device=dev)
    _dev(xd, "xd")
    B = sum(int(t.shape[0]) for t in seg_x)
    _need(row_of, "row_of", shape=(B, K))
    if xd.dtype != _TORCH[xd_code]:
        raise ValueError(f"xd must be {_TORCH[xd_code]} (got {xd.dtype})")
    _need(xd, "xd", numel=cap_rows * H)
    if xd_code == MOE_FP8_E4M3:
        _dev(xd_scales, "xd_scales", torch.float32)
        _need(xd_scales, "xd_scales", numel=cap_rows * (-(-H // FP8_BLOCK)))
    ptrs = (ctypes.c_void_p * len(seg_x))(*[s.data_ptr() for s in seg_x])
    rows = (ctypes.c_int32 * len(seg_x))(*[s.shape[0] for s in seg_x])
    _check(lib().moe_dispatch(ctypes.cast(ptrs, ctypes.c_void_p), ctypes.cast(rows, ctypes.c_void_p),
                              len(seg_x), _DT[x_dt], H, _ptr(row_of), K, _ptr(xd), xd_code,
                              _ptr(xd_scales), cap_rows, _stream(stream)))
    return xd, xd_scales


def moe_ffn_workspace_bytes(cap_rows: int, I: int, act_dtype) -> int:
    return int(lib().moe_ffn_workspace_bytes(cap_rows, I, _dtype_code(act_dtype)))


def moe_weight_ld(cols: int, w_dtype) -> int:
    """Row pitch (elements) of packed weights with rows of ``cols`` elements."""
    ld = int(lib().moe_weight_ld(int(cols), _dtype_code(w_dtype)))
    if ld < 0:
        raise ValueError(f"no packed pitch for cols={cols}, dtype={w_dtype}")
    return ld


def moe_packed_weight_bytes(E_local: int, rows: int, cols: int, w_dtype) -> int:
    return int(lib().moe_packed_weight_bytes(E_local, rows, cols, _dtype_code(w_dtype)))


def moe_pack_weights(w, out=None, stream=None):
    """w (E_local, rows, cols) -> (E_local, rows, moe_weight_ld(cols)), rows
    unchanged and the padding zero: the layout the FFN calls read when given
    weights with the packed pitch (results identical to the dense weights)."""
    _dev(w, "w", ndim=3)
    E_loc, rows, cols = w.shape
    code = _DT[w.dtype]
    ld = moe_weight_ld(cols, code)
    if out is None:
        out = torch.empty((E_loc, rows, ld), dtype=w.dtype, device=w.device)
    _dev(out, "out", w.dtype)
    _need(out, "out", shape=(E_loc, rows, ld))
    _check(lib().moe_pack_weights(_ptr(w), E_loc, rows, cols, code, _ptr(out), _stream(stream)))
    return out


def _w_packed(w, in_dim, act, name):
    """Layout of weight tensor w (E_local, out, last): False if last is the
    input dim (dense), True if it is the packed pitch, None when the packed
    pitch equals the input dim (both layouts are the same)."""
    ld = moe_weight_ld(in_dim, act)
    last = w.shape[2]
    if last == in_dim:
        return None if ld == in_dim else False
    if last == ld:
        return True
    raise ValueError(f"{name} must have {in_dim} columns (dense) or {ld} (packed), got {last}")


def _pack_flag(*layouts):
    """MOE_W_PACKED if the call's weights are packed; all of one call's
    weights share one layout."""
    seen = {x for x in layouts if x is not None}
    if len(seen) > 1:
        raise ValueError("the weights of one call must be all packed or all dense")
    return MOE_W_PACKED if seen == {True} else 0


def _rows_arg(rows, cap_per_expert, E_loc, n_rows):
    """(pointer tensor, third int argument) of the row description: offsets
    (E_loc+1) of the contiguous layout, or m (E_loc) of the masked one."""
    _dev(rows, "offsets" if cap_per_expert is None else "m", torch.int32, 1)
    if cap_per_expert is None:
        return n_rows
    if n_rows != E_loc * cap_per_expert:
        raise ValueError(f"masked layout needs E_loc * cap_per_expert = {E_loc * cap_per_expert} rows, "
                         f"got {n_rows}")
    return int(cap_per_expert)


def _check_ffn(a, a_scales, rows, cap_per_expert, E_loc, Kdim, cap, act, **tensors):
    """Shapes of the FFN operands: the activation rows (cap, Kdim) [+ fp8
    scales], the row description (offsets E_loc + 1, or m E_loc), and each
    named (tensor, shape or minimum element count) pair."""
    if a.shape[1] != Kdim:
        raise ValueError(f"activations must have {Kdim} columns (got {a.shape[1]})")
    _need(rows, "offsets" if cap_per_expert is None else "m",
          numel=E_loc + 1 if cap_per_expert is None else E_loc)
    if act == MOE_FP8_E4M3:
        if a_scales is None:
            raise ValueError("fp8 activations need their block scales")
        _dev(a_scales, "activation scales", torch.float32)
        _need(a_scales, "activation scales", numel=cap * (-(-Kdim // FP8_BLOCK)))
    for name, (t, want) in tensors.items():
        if t is None:
            continue
        _dev(t, name)
        if isinstance(want, tuple):
            _need(t, name, shape=want)
        else:
            _need(t, name, numel=want)


def _w_code(act, w_scales_pow2):
    """Weight dtype code: fp8 weights whose block scales are all powers of two
    are declared as MOE_FP8_E4M3_PO2."""
    if w_scales_pow2 and act != MOE_FP8_E4M3:
        raise ValueError("w_scales_pow2 applies to fp8 weights only")
    return MOE_FP8_E4M3_PO2 if w_scales_pow2 else act


def moe_ffn_gate_up(xd, xd_scales, offsets, w_gate, w_up, w_gate_scales=None, w_up_scales=None,
                    h=None, h_scales=None, expected_rows=0, stream=None, cap_per_expert=None,
                    w_scales_pow2=False):
    """h = silu(Xd Wg^T) * (Xd Wu^T) per local expert -> (cap_rows, I) [+ scales].
    expected_rows: rows a local expert is expected to get (tile-shape hint only).
    With cap_per_expert given, ``offsets`` is the masked layout's m and the call
    is moe_ffn_gate_up_masked.  w_scales_pow2: the fp8 weight scales are all
    powers of two (weight dtype MOE_FP8_E4M3_PO2)."""
    _dev(xd, "xd", ndim=2)
    _dev(w_gate, "w_gate", xd.dtype, 3)
    _dev(w_up, "w_up", xd.dtype, 3)
    E_loc, I, H = w_gate.shape[0], w_gate.shape[1], xd.shape[1]
    cap = xd.shape[0]
    third = _rows_arg(offsets, cap_per_expert, E_loc, cap)
    act = _DT[xd.dtype]
    packed = _pack_flag(_w_packed(w_gate, H, act, "w_gate"))
    if h is None:
        h = torch.empty((cap, I), dtype=xd.dtype, device=xd.device)
    if act == MOE_FP8_E4M3 and h_scales is None:
        h_scales = torch.empty((cap, -(-I // FP8_BLOCK)), dtype=torch.float32, device=xd.device)
    if h.dtype != xd.dtype:
        raise ValueError(f"h must be {xd.dtype} (got {h.dtype})")
    nbH, nbI = -(-H // FP8_BLOCK), -(-I // FP8_BLOCK)
    fp8 = act == MOE_FP8_E4M3
    _check_ffn(xd, xd_scales, offsets, cap_per_expert, E_loc, H, cap, act,
               w_up=(w_up, tuple(w_gate.shape)), h=(h, cap * I),
               h_scales=(h_scales if fp8 else None, cap * nbI),
               w_gate_scales=(w_gate_scales if fp8 else None, (E_loc, I, nbH)),
               w_up_scales=(w_up_scales if fp8 else None, (E_loc, I, nbH)))
    fn = lib().moe_ffn_gate_up if cap_per_expert is None else lib().moe_ffn_gate_up_masked
    _check(fn(_ptr(xd), _ptr(xd_scales), _ptr(offsets), E_loc, third, H, I, act,
              _ptr(w_gate), _ptr(w_up), _ptr(w_gate_scales), _ptr(w_up_scales),
              _w_code(act, w_scales_pow2) | packed, _ptr(h), _ptr(h_scales), int(expected_rows),
              _stream(stream)))
    return h, h_scales


def _y_dtype_for(act):
    return torch.float32 if act == MOE_F32 else torch.bfloat16


def moe_ffn_down(h, h_scales, offsets, w_down, w_down_scales=None, y=None, y_dtype=None,
                 expected_rows=0, stream=None, cap_per_expert=None, w_scales_pow2=False):
    """y = h Wd^T per local expert -> (cap_rows, H).  cap_per_expert and
    w_scales_pow2: as in moe_ffn_gate_up (moe_ffn_down_masked)."""
    _dev(h, "h", ndim=2)
    _dev(w_down, "w_down", h.dtype, 3)
    E_loc, H, I = w_down.shape[0], w_down.shape[1], h.shape[1]
    cap = h.shape[0]
    third = _rows_arg(offsets, cap_per_expert, E_loc, cap)
    act = _DT[h.dtype]
    packed = _pack_flag(_w_packed(w_down, I, act, "w_down"))
    y_dtype = _y_dtype_for(act) if y_dtype is None else y_dtype
    if y is None:
        y = torch.empty((cap, H), dtype=y_dtype, device=h.device)
    fp8 = act == MOE_FP8_E4M3
    _check_ffn(h, h_scales, offsets, cap_per_expert, E_loc, I, cap, act, y=(y, cap * H),
               w_down_scales=(w_down_scales if fp8 else None, (E_loc, H, -(-I // FP8_BLOCK))))
    fn = lib().moe_ffn_down if cap_per_expert is None else lib().moe_ffn_down_masked
    _check(fn(_ptr(h), _ptr(h_scales), _ptr(offsets), E_loc, third, H, I, act,
              _ptr(w_down), _ptr(w_down_scales), _w_code(act, w_scales_pow2) | packed, _ptr(y), _DT[y.dtype],
              int(expected_rows), _stream(stream)))
    return y


def moe_grouped_ffn(xd, xd_scales, offsets, w_gate, w_up, w_down, w_gate_scales=None,
                    w_up_scales=None, w_down_scales=None, y=None, y_dtype=None, ws=None,
                    expected_rows=0, stream=None, cap_per_expert=None, w_scales_pow2=False):
    """Both FFN stages with h held in the workspace ``ws``.  cap_per_expert
    and w_scales_pow2: as in moe_ffn_gate_up (moe_grouped_ffn_masked)."""
    _dev(xd, "xd", ndim=2)
    for n, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _dev(w, n, xd.dtype, 3)
    E_loc, I, H = w_gate.shape[0], w_gate.shape[1], xd.shape[1]
    cap = xd.shape[0]
    third = _rows_arg(offsets, cap_per_expert, E_loc, cap)
    act = _DT[xd.dtype]
    packed = _pack_flag(_w_packed(w_gate, H, act, "w_gate"), _w_packed(w_down, I, act, "w_down"))
    y_dtype = _y_dtype_for(act) if y_dtype is None else y_dtype
    if y is None:
        y = torch.empty((cap, H), dtype=y_dtype, device=xd.device)
    need = moe_ffn_workspace_bytes(cap, I, act)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=xd.device)
    fp8 = act == MOE_FP8_E4M3
    nbH, nbI = -(-H // FP8_BLOCK), -(-I // FP8_BLOCK)
    _check_ffn(xd, xd_scales, offsets, cap_per_expert, E_loc, H, cap, act,
               w_up=(w_up, tuple(w_gate.shape)), w_down=(w_down, (E_loc, H, w_down.shape[2])),
               y=(y, cap * H),
               w_gate_scales=(w_gate_scales if fp8 else None, (E_loc, I, nbH)),
               w_up_scales=(w_up_scales if fp8 else None, (E_loc, I, nbH)),
               w_down_scales=(w_down_scales if fp8 else None, (E_loc, H, nbI)))
    fn = lib().moe_grouped_ffn if cap_per_expert is None else lib().moe_grouped_ffn_masked
    _check(fn(_ptr(xd), _ptr(xd_scales), _ptr(offsets), E_loc, third, H, I, act,
              _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(w_gate_scales),
              _ptr(w_up_scales), _ptr(w_down_scales), _w_code(act, w_scales_pow2) | packed, _ptr(y),
              _DT[y.dtype], _ptr(ws), ws.numel() * ws.element_size(),
              int(expected_rows), _stream(stream)))
    return y


def moe_ffn_gate_up_masked(xd, xd_scales, m, cap_per_expert, w_gate, w_up, **kw):
    """moe_ffn_gate_up over the masked layout (rows [j*cap_per_expert, +m[j]))."""
    return moe_ffn_gate_up(xd, xd_scales, m, w_gate, w_up, cap_per_expert=cap_per_expert, **kw)


def moe_ffn_down_masked(h, h_scales, m, cap_per_expert, w_down, **kw):
    """moe_ffn_down over the masked layout."""
    return moe_ffn_down(h, h_scales, m, w_down, cap_per_expert=cap_per_expert, **kw)


def moe_grouped_ffn_masked(xd, xd_scales, m, cap_per_expert, w_gate, w_up, w_down, **kw):
    """moe_grouped_ffn over the masked layout."""
    return moe_grouped_ffn(xd, xd_scales, m, w_gate, w_up, w_down, cap_per_expert=cap_per_expert, **kw)


def moe_combine(y, row_of, topk_w, out=None, out_dtype=None, stream=None):
    """out[t] = sum_k topk_w[t,k] * y[row_of[t,k]] over local slots -> (B, H)."""
    _dev(y, "y", ndim=2)
    _dev(row_of, "row_of", torch.int32, 2)
    _dev(topk_w, "topk_w", torch.float32, 2)
    B, K = row_of.shape
    H = y.shape[1]
    if out is None:
        out = torch.empty((B, H), dtype=y.dtype if out_dtype is None else out_dtype, device=y.device)
    _dev(out, "out")
    _need(topk_w, "topk_w", shape=(B, K))
    _need(out, "out", numel=B * H)
    _check(lib().moe_combine(_ptr(y), _DT[y.dtype], y.shape[0], _ptr(row_of), _ptr(topk_w), B, K, H,
                             _ptr(out), _DT[out.dtype], _stream(stream)))
    return out


from .layer import MoELayer  # noqa: E402  (uses the functions above)
