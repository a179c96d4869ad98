"""One GPU's share of the expert-parallel MoE layer, with its buffers
allocated once (capacity-sized, so every call has static sizes and no host
synchronisation, the property the Moreh report's "Using HIP Graphs" section
asks of an EP decode step).

    route -> layout -> dispatch -> gate/up (+SwiGLU) -> down -> combine

Every stage is one call into libmoeep; this class only owns the buffers
and orders the calls on one stream.
"""
from __future__ import annotations

import torch

from . import (FP8_BLOCK, moe_combine, moe_dispatch, moe_ffn_down, moe_ffn_gate_up,
               moe_layout, moe_layout_masked, moe_layout_workspace_bytes, moe_route,
               moe_route_mapped, moe_route_shared)

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}


class MoELayer:
    """Buffers and stage order for one layer shape.

    seg_rows: tokens per simulated source segment (T = sum); E routed experts,
    K per token; H hidden, I expert intermediate; local experts
    [e_begin, e_end); act_dtype stores Xd and h ('f32' | 'bf16' | 'fp8');
    y_dtype / out_dtype store the expert outputs and the combined rows.
    layout: 'contiguous' (rows of the local experts back to back, cap_rows
    rows, default T*K) or 'masked' (a fixed block of cap_per_expert rows per
    local expert, default T -- no slot can be dropped).
    n_shared: always-on shared experts (every token, gate 1), run as experts
    E, E+1, ... of the same grouped FFN; the local range must end at E and the
    weights hold the shared experts after the routed ones.  self.E, self.K
    and self.e_end then count them (self.E_routed, self.K_routed do not).
    """

    def __init__(self, seg_rows, E, K, H, I, e_begin, e_end, act_dtype, y_dtype, out_dtype,
                 device="cuda", cap_rows=None, layout="contiguous", cap_per_expert=None, n_shared=0):
        self.seg_rows = tuple(int(b) for b in seg_rows)
        self.T = sum(self.seg_rows)
        self.n_shared = int(n_shared)
        if self.n_shared and e_end != E:
            raise ValueError("shared experts need the local range to end at E")
        self.E_routed, self.K_routed = E, K
        E, K, e_end = E + self.n_shared, K + self.n_shared, e_end + self.n_shared
        self.E, self.K, self.H, self.I = E, K, H, I
        self.e_begin, self.e_end = e_begin, e_end
        self.E_loc = e_end - e_begin
        self.act_dtype, self.y_dtype, self.out_dtype = act_dtype, y_dtype, out_dtype
        if layout not in ("contiguous", "masked"):
            raise ValueError(f"unknown layout {layout!r}")
        self.masked = layout == "masked"
        self.cap_e = (max(self.T, 1) if cap_per_expert is None else int(cap_per_expert)) if self.masked else None
        if self.masked:
            self.cap = self.E_loc * self.cap_e
        else:
            self.cap = self.T * K if cap_rows is None else int(cap_rows)
        # rows a routed local expert gets under balanced routing: the FFN tile-shape hint
        self.expected_rows = max(1, (self.T * self.K_routed) // self.E_routed)
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        T, cap = self.T, max(self.cap, 1)
        self.topk_ids = torch.empty((T, K), **i32)
        self.topk_w = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(self.E_loc + 1, **i32)     # contiguous: offsets; masked: m (E_loc)
        self.row_of = torch.empty((T, K), **i32)
        self.src_of = torch.empty(cap, **i32)
        self.layout_ws = torch.empty(max(moe_layout_workspace_bytes(T, K, E), 256),
                                     dtype=torch.uint8, device=dev)
        act = _TORCH[act_dtype]
        self.xd = torch.empty((cap, H), dtype=act, device=dev)
        self.h = torch.empty((cap, I), dtype=act, device=dev)
        fp8 = act_dtype == "fp8"
        self.xd_scales = torch.empty((cap, -(-H // FP8_BLOCK)), dtype=torch.float32, device=dev) if fp8 else None
        self.h_scales = torch.empty((cap, -(-I // FP8_BLOCK)), dtype=torch.float32, device=dev) if fp8 else None
        self.y = torch.empty((cap, H), dtype=_TORCH[y_dtype], device=dev)
        self.out = torch.empty((T, H), dtype=_TORCH[out_dtype], device=dev)
        # placement map (E,) int32 on the device, logical -> physical expert id; when
        # set, routing emits physical ids and [e_begin, e_end) is a physical range
        self.expert_map = None

    # individual stages (each one library call) ---------------------------------
    def route(self, logits, stream=None):
        if self.n_shared:
            if self.expert_map is not None:
                raise ValueError("a placement map with shared experts is not supported")
            moe_route_shared(logits, self.K_routed, self.n_shared, self.topk_ids, self.topk_w,
                             stream=stream)
        elif self.expert_map is None:
            moe_route(logits, self.K, self.topk_ids, self.topk_w, stream=stream)
        else:
            moe_route_mapped(logits, self.K, self.expert_map, self.topk_ids, self.topk_w, stream=stream)

    def layout(self, stream=None):
        if self.masked:
            moe_layout_masked(self.topk_ids, self.E, self.e_begin, self.e_end, self.cap_e, self.counts,
                              self.offsets[:self.E_loc], self.row_of, self.src_of, self.layout_ws,
                              stream=stream)
        else:
            moe_layout(self.topk_ids, self.E, self.e_begin, self.e_end, self.cap, self.counts,
                       self.offsets, self.row_of, self.src_of, self.layout_ws, stream=stream)

    @property
    def rows(self):
        """The FFN's row description: offsets (contiguous) or m (masked)."""
        return self.offsets[:self.E_loc] if self.masked else self.offsets

    def dispatch(self, x_segments, stream=None):
        moe_dispatch(x_segments, self.row_of, self.cap, self.act_dtype, self.xd, self.xd_scales,
                     stream=stream)

    def gate_up(self, w, stream=None):
        moe_ffn_gate_up(self.xd, self.xd_scales, self.rows, w["gate"], w["up"],
                        w.get("gate_scale"), w.get("up_scale"), self.h, self.h_scales,
                        expected_rows=self.expected_rows, stream=stream, cap_per_expert=self.cap_e,
                        w_scales_pow2=bool(w.get("scales_pow2", False)))

    def down(self, w, stream=None):
        moe_ffn_down(self.h, self.h_scales, self.rows, w["down"], w.get("down_scale"), self.y,
                     expected_rows=self.expected_rows, stream=stream, cap_per_expert=self.cap_e,
                     w_scales_pow2=bool(w.get("scales_pow2", False)))

    def combine(self, stream=None):
        moe_combine(self.y, self.row_of, self.topk_w, self.out, stream=stream)

    def stages(self, x_segments, logits, w):
        """(name, thunk) pairs of the six calls, in order."""
        return [("route", lambda s=None: self.route(logits, s)),
                ("layout", lambda s=None: self.layout(s)),
                ("dispatch", lambda s=None: self.dispatch(x_segments, s)),
                ("ffn_gate_up", lambda s=None: self.gate_up(w, s)),
                ("ffn_down", lambda s=None: self.down(w, s)),
                ("combine", lambda s=None: self.combine(s))]

    def forward(self, x_segments, logits, w, stream=None):
        for _, run in self.stages(x_segments, logits, w):
            run(stream)
        return self.out


class MicroBatchedLayer:
    """The layer over two micro-batches on two streams (Moreh report,
    compute-communication overlapping: split the batch in two so one
    micro-batch's dispatch/combine runs under the other's expert GEMMs).

    The tokens are split at a segment boundary (or, for one segment, at its
    middle row).  Stream 0 runs micro-batch A's six calls; stream 1 runs B's
    route, layout and dispatch at once, starts B's GEMMs after A's, and B's
    combine follows them, so A's combine overlaps B's GEMMs and B's dispatch
    overlaps A's.  Per-token results equal the single-batch layer's bit for
    bit (every row is computed by the same kernels in the same order).
    Both streams have the default priority.
    """

    def __init__(self, seg_rows, *args, **kw):
        seg_rows = [int(b) for b in seg_rows]
        if len(seg_rows) > 1:
            cut = len(seg_rows) // 2
            self.parts = (seg_rows[:cut], seg_rows[cut:])
        else:
            half = seg_rows[0] // 2
            self.parts = ([half], [seg_rows[0] - half])
        if min(sum(p) for p in self.parts) < 1:
            raise ValueError("each micro-batch needs at least one token")
        self.a = MoELayer(self.parts[0], *args, **kw)
        self.b = MoELayer(self.parts[1], *args, **kw)
        self.T = self.a.T + self.b.T
        # the whole batch's tile-shape hint, so both halves use the single-batch kernels
        self.a.expected_rows = self.b.expected_rows = max(
            1, (self.T * self.a.K_routed) // self.a.E_routed)
        self.side = torch.cuda.Stream(device=self.a.out.device)   # default priority
        self._ev_a_ffn = torch.cuda.Event()
        self._ev_b_done = torch.cuda.Event()
        self._ev_start = torch.cuda.Event()

    def split_inputs(self, x_segments, logits):
        """(x segments, logits) of each micro-batch, as views of the inputs."""
        xs = list(x_segments)
        Ta = self.a.T
        if len(xs) > 1:
            cut = len(self.parts[0])
            xa, xb = xs[:cut], xs[cut:]
        else:
            xa, xb = [xs[0][:Ta]], [xs[0][Ta:]]
        return (xa, logits[:Ta]), (xb, logits[Ta:])

    def forward(self, x_segments, logits, w):
        """Enqueue both micro-batches; returns (out_a, out_b) (token order: A then B)."""
        (xa, la), (xb, lb) = self.split_inputs(x_segments, logits)
        main = torch.cuda.current_stream()
        self._ev_start.record(main)
        self.side.wait_event(self._ev_start)
        a, b = self.a, self.b
        a.route(la, main)
        a.layout(main)
        a.dispatch(xa, main)
        b.route(lb, self.side)
        b.layout(self.side)
        b.dispatch(xb, self.side)
        a.gate_up(w, main)
        a.down(w, main)
        self._ev_a_ffn.record(main)
        a.combine(main)
        self.side.wait_event(self._ev_a_ffn)
        b.gate_up(w, self.side)
        b.down(w, self.side)
        b.combine(self.side)
        self._ev_b_done.record(self.side)
        main.wait_event(self._ev_b_done)
        return a.out, b.out
