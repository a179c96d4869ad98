"""Plain CPU oracle of the single-GPU expert-parallel MoE layer.

Test infrastructure only.  Only ``tests/``, the package smoke check and the
bench's CPU-baseline leg may import this module; the product path never does.

What the layer computes, and where the pages state it:

* route  -- per token, the K experts with the largest router logits
  ("Anatomy of a high-performance EP kernel", section "What we have to do",
  the router figure: a (B_i, E) logit tensor reduced to a (B_i, K) index
  tensor; the same figure in the Chinese translation of that post carries the
  four worked rows t0..t3).  The gate weights are a softmax over the selected
  logits (equivalently, the full softmax renormalised over the K picks); the
  pages never state the gate function, so this is a reading.
* layout -- group the routed (token, slot) pairs by expert: a histogram,
  an exclusive prefix sum and a permutation ("Anatomy ...", section
  "Dispatch": every expert receives a different number of tokens and the
  grouped GEMM runs over one row set per expert; SGLang "Expert Parallelism",
  "Framework Overview" flow diagram: pre-permute before the grouped GEMM).
* dispatch -- gather the routed token rows into one dense, expert-contiguous
  buffer ("Anatomy ...", section "Dispatch").
* grouped FFN -- per expert a small feed-forward network (Moreh report,
  "Overview": experts are small FFN layers); its SwiGLU form, gate/up H->I and
  down I->H, is the reading used throughout.
* combine -- return each expert output to its token and reduce the K
  contributions ("Anatomy ...", the paragraph after the router figure: run the
  expert GEMM where the activations landed, then bring the results home;
  SGLang "Framework Overview": post-permute then combine).  The reduction is
  the gate-weighted sum.

Floating point is fp64 throughout; values are rounded only where the layer
stores a tensor in a narrower type (x, Xd, h, y, out).  Integer outputs are
exact.
"""
from __future__ import annotations

import numpy as np

from . import numerics as nx


# ----------------------------------------------------------------------------
# route
# ----------------------------------------------------------------------------
def route(logits, K: int):
    """Top-K experts per token and their gate weights.

    logits: (B, E) finite floats.  Returns ids (B, K) int32 and gates (B, K)
    fp64.  Slot k holds the k-th largest logit; equal logits go to the lower
    expert id first (a stable descending sort).  gates[t] = softmax over the K
    selected logits, shifted by their maximum before exponentiation.
    """
    lg = np.asarray(logits, dtype=np.float64)
    if lg.ndim != 2:
        raise ValueError("logits must be (B, E)")
    B, E = lg.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    if not np.all(np.isfinite(lg)):
        raise ValueError("non-finite logits are outside the method")
    # stable sort of the negated logits keeps equal logits in ascending id order
    order = np.argsort(-lg, axis=1, kind="stable")
    ids = order[:, :K].astype(np.int32)
    sel = np.take_along_axis(lg, order[:, :K], axis=1)
    ex = np.exp(sel - sel[:, :1])
    gates = ex / ex.sum(axis=1, keepdims=True)
    return ids, gates


# ----------------------------------------------------------------------------
# layout
# ----------------------------------------------------------------------------
def route_shared(logits, K: int, n_shared: int):
    """Routing with n_shared always-on (shared) experts.

    Moreh report, "Overview": besides the routed experts, a shared expert runs
    for every token regardless of routing; its section on library
    optimisations merges the shared expert's GEMMs with others (horizontal
    fusion).  Reading: the shared experts are experts E, E+1, ... that every
    token selects with gate 1 (their output is added unweighted), appended
    after the K routed slots, so the rest of the layer runs them as ordinary
    expert groups.  Returns ids (T, K + n_shared), gates (T, K + n_shared).
    """
    ids, gates = route(logits, K)
    T, E = np.asarray(logits).shape
    extra = np.tile(np.arange(E, E + n_shared, dtype=np.int32), (T, 1))
    return (np.concatenate([ids, extra], axis=1).astype(np.int32),
            np.concatenate([gates, np.ones((T, n_shared))], axis=1))


def layout(ids, E: int, e_begin: int, e_end: int, cap: int):
    """Per-expert counts, offsets and the (token, slot) <-> row permutation.

    counts[e]   number of (t, k) with ids[t, k] == e, over all E experts.
    offsets     exclusive prefix sum of counts over the local experts
                [e_begin, e_end), with the total appended (length E_loc + 1).
    row_of[t,k] destination row of slot (t, k) in the expert-contiguous
                buffer, -1 when its expert is not local.
    src_of[r]   flattened slot index t*K + k that row r holds; -1 for the
                padding rows [offsets[-1], cap).
    Rows of one expert are ordered by (t, k) ascending.
    """
    ids = np.asarray(ids)
    B, K = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    E_loc = e_end - e_begin
    offsets = np.zeros(E_loc + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts[e_begin:e_end])
    R = int(offsets[-1])
    if cap < R:
        raise ValueError("cap smaller than the number of local rows")
    local = (flat >= e_begin) & (flat < e_end)
    slots = np.nonzero(local)[0]                       # ascending slot order
    perm = np.argsort(flat[slots], kind="stable")      # stable: keeps (t, k) order
    src_of = np.full(cap, -1, dtype=np.int32)
    src_of[:R] = slots[perm]
    row_of = np.full(B * K, -1, dtype=np.int32)
    row_of[src_of[:R]] = np.arange(R, dtype=np.int32)
    return {"counts": counts, "offsets": offsets,
            "row_of": row_of.reshape(B, K), "src_of": src_of}


def layout_masked(ids, E: int, e_begin: int, e_end: int, cap_e: int):
    """Fixed-capacity ("masked") layout of the routed slots.

    SGLang "Expert Parallelism", MoE-runner backend table: the grouped GEMM
    takes a contiguous layout for prefill and a masked layout for decode; the
    same page's dispatch paragraph pairs the low-latency (decode) mode with
    CUDA-graph compatibility.  The page gives no further detail; the reading
    used here: local expert j owns the fixed row block [j*cap_e, (j+1)*cap_e)
    and a count m[j] of valid rows (the mask), so every size is static.

    counts[e]   number of (t, k) with ids[t, k] == e, over all E experts.
    m[j]        valid rows of local expert j = min(counts[e_begin + j], cap_e).
    row_of[t,k] j*cap_e + (rank of (t, k) among the slots routed to local
                expert j, in (t, k) order), or -1 when the expert is not local
                or the rank is >= cap_e (the slot is dropped).
    src_of[r]   slot index t*K + k held by row r, -1 for unused rows.
    """
    ids = np.asarray(ids)
    B, K = ids.shape
    E_loc = e_end - e_begin
    counts = np.zeros(E, dtype=np.int32)
    m = np.zeros(E_loc, dtype=np.int32)
    row_of = np.full((B, K), -1, dtype=np.int32)
    src_of = np.full(E_loc * cap_e, -1, dtype=np.int32)
    for t in range(B):                     # slots in (t, k) order
        for k in range(K):
            e = int(ids[t, k])
            if not 0 <= e < E:
                continue
            rank = int(counts[e])
            counts[e] += 1
            if e_begin <= e < e_end and rank < cap_e:
                j = e - e_begin
                row_of[t, k] = j * cap_e + rank
                src_of[j * cap_e + rank] = t * K + k
                m[j] += 1
    return {"counts": counts, "m": m, "row_of": row_of, "src_of": src_of}


# ----------------------------------------------------------------------------
# dispatch
# ----------------------------------------------------------------------------
def dispatch(x, row_of, n_rows: int, act: str):
    """Dense expert-contiguous input: Xd[row_of[t, k]] = x[t].

    x: (T, H) values already on the x storage grid.  act selects the storage
    of Xd: 'f32' / 'bf16' copy the row unchanged (x must already be on that
    grid); 'fp8' quantises each token row once (block-wise, see numerics) and
    every one of its K copies holds the same codes and scales.
    Returns (xd, xd_scales) with xd of shape (n_rows, H) (codes for fp8) and
    xd_scales (n_rows, ceil(H/128)) fp32 for fp8, else None.
    """
    x = np.asarray(x, dtype=np.float64)
    row_of = np.asarray(row_of)
    T, H = x.shape
    if act == "fp8":
        src, scales_src = nx.quantize_fp8_blocks(x)
    elif act in ("f32", "bf16"):
        src, scales_src = x, None
    else:
        raise ValueError(act)
    xd = np.zeros((n_rows, H), dtype=np.float64)
    xs = None if scales_src is None else np.zeros((n_rows, scales_src.shape[1]), np.float32)
    for t in range(T):
        for r in row_of[t]:
            if r >= 0:
                xd[r] = src[t]
                if xs is not None:
                    xs[r] = scales_src[t]
    return xd, xs


# ----------------------------------------------------------------------------
# expert FFN
# ----------------------------------------------------------------------------
def silu(z):
    """z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(X, Wg, Wu, Wd, h_dtype: str, y_dtype: str):
    """One expert's SwiGLU FFN on the rows routed to it.

    X (n, H) values the expert sees (dequantised when stored as fp8);
    Wg, Wu (I, H) and Wd (H, I) weight values (dequantised likewise), laid
    out (out, in) so that g = X Wg^T.
    g = X Wg^T, u = X Wu^T, h = silu(g) * u stored as h_dtype,
    y = h Wd^T stored as y_dtype.  Returns y in fp64 on the y grid.
    """
    X = np.asarray(X, dtype=np.float64)
    g = X @ np.asarray(Wg, dtype=np.float64).T
    u = X @ np.asarray(Wu, dtype=np.float64).T
    h = silu(g) * u
    hr = nx.round_act(h, h_dtype)
    if h_dtype == "fp8":
        hr = nx.dequantize_fp8_blocks(*hr)
    y = hr @ np.asarray(Wd, dtype=np.float64).T
    return nx.round_act(y, y_dtype)


def grouped_ffn(xd, offsets, weights_of, h_dtype: str, y_dtype: str):
    """Run each local expert's FFN on its contiguous row range.

    xd (R, H) dequantised values; offsets (E_loc + 1); weights_of(e) returns
    the dequantised (Wg, Wu, Wd) of local expert e.  Returns y (R, H).
    Empty experts contribute nothing.
    """
    xd = np.asarray(xd, dtype=np.float64)
    offsets = np.asarray(offsets)
    y = np.zeros_like(xd)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = expert_ffn(xd[a:b], *weights_of(e), h_dtype, y_dtype)
    return y


def grouped_ffn_masked(xd, m, cap_e: int, weights_of, h_dtype: str, y_dtype: str):
    """The grouped FFN over a masked layout: local expert j runs on rows
    [j*cap_e, j*cap_e + m[j]); the other rows of y stay zero."""
    xd = np.asarray(xd, dtype=np.float64)
    y = np.zeros_like(xd)
    for j, n in enumerate(np.asarray(m)):
        a = j * cap_e
        if n > 0:
            y[a:a + n] = expert_ffn(xd[a:a + n], *weights_of(j), h_dtype, y_dtype)
    return y


# ----------------------------------------------------------------------------
# combine
# ----------------------------------------------------------------------------
def combine(y, row_of, gates, out_dtype: str):
    """out[t] = sum over local slots k of gates[t, k] * y[row_of[t, k]],
    stored as out_dtype.  Tokens with no local slot get 0."""
    y = np.asarray(y, dtype=np.float64)
    row_of = np.asarray(row_of)
    gates = np.asarray(gates, dtype=np.float64)
    T, K = row_of.shape
    out = np.zeros((T, y.shape[1]), dtype=np.float64)
    for t in range(T):
        for k in range(K):
            r = row_of[t, k]
            if r >= 0:
                out[t] += gates[t, k] * y[r]
    return nx.round_act(out, out_dtype)


# ----------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------
def layer(x, logits, K, E, e_begin, e_end, weights_of, act, y_dtype, out_dtype,
          gates_dtype="f32", n_shared=0):
    """route -> layout -> dispatch -> grouped FFN -> combine on one GPU's share.

    x (T, H) token rows (values on their storage grid), logits (T, E).
    weights_of(e) gives local expert e's dequantised weights.  Gates are
    stored as fp32 before use (gates_dtype) as the layer hands them between
    steps in fp32.  With n_shared > 0 the shared experts E.. are appended to
    the routing (route_shared) and to the local range, which must then end
    at E.  Returns a dict with every intermediate.
    """
    if n_shared:
        if e_end != E:
            raise ValueError("shared experts need the local range to end at E")
        ids, gates = route_shared(logits, K, n_shared)
        K, E, e_end = K + n_shared, E + n_shared, E + n_shared
    else:
        ids, gates = route(logits, K)
    gates_s = nx.round_act(gates, gates_dtype)
    T = np.asarray(x).shape[0]
    lay = layout(ids, E, e_begin, e_end, T * K)
    R = int(lay["offsets"][-1])
    xd, xs = dispatch(x, lay["row_of"], R, act)
    xd_val = nx.dequantize_fp8_blocks(xd, xs) if act == "fp8" else xd
    y = grouped_ffn(xd_val, lay["offsets"], weights_of, act, y_dtype)
    out = combine(y, lay["row_of"], gates_s, out_dtype)
    return {"ids": ids, "gates": gates, **lay, "xd": xd, "xd_scales": xs,
            "y": y, "out": out}
