"""Bench of the single-GPU expert-parallel MoE layer on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-others]

One step is one pass of the whole path -- route, layout, dispatch, gate/up
GEMM + SwiGLU, down GEMM, combine -- over one batch of seeded synthetic
input already resident in HBM.  The headline workload is the DeepSeek-V3
shaped prefill step (T=8192, E=256, K=8, H=7168, I=2048, bf16), the largest
configuration and the one the grouped-GEMM bar applies to.

Timed steps run cold: they rotate over enough independent sets of input and
activation buffers (x, logits, routing, Xd, h, y, out) that the sets together
exceed twice the 256 MB Infinity Cache, so no step finds the previous
step's activations in cache (a producer's output inside one step still may,
as in a real layer).  The expert weights are shared and far larger than the
cache.  A second, warm pass repeats the steps on one buffer set and is
reported beside them.  Each stage is bracketed by HIP events on the launch
stream, so per-kernel durations, algorithmic GB/s and TFLOP/s come from the
same run.

Prints one JSON line (rank 0).  The other workloads (toy, decode, EP-share,
GPT-OSS) are timed the same way after the headline and reported as
sub-objects of that line unless --no-others is given.  A CPU baseline --
the oracle as it stands, timed on a bounded sample of the headline workload
on the host cores -- is included unless --no-cpu-baseline is given.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0                     # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
ESIZE = {"f32": 4, "bf16": 2, "fp8": 1}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill", choices=sorted(wl.CONFIGS))
    ap.add_argument("--no-others", action="store_true",
                    help="time only --workload (no sub-objects for the other workloads)")
    ap.add_argument("--cold-mb", type=int, default=512,
                    help="rotate buffer sets until they exceed this many MB (0: one set, warm only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dense-weights", action="store_true",
                    help="feed the FFN the weights in their dense (out, in) layout instead of packing them "
                         "once (untimed) to the library's padded row pitch")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0,
                    help="target CPU seconds for the oracle sample")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for counter calibration)")
    ap.add_argument("--layout", default="contiguous", choices=["contiguous", "masked"],
                    help="expert row layout: contiguous (offsets) or masked (fixed block per expert)")
    ap.add_argument("--cap-per-expert", type=int, default=0,
                    help="masked layout: rows per expert block (default T, nothing dropped)")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step as a HIP graph and time its replays")
    ap.add_argument("--shared-experts", type=int, default=0,
                    help="always-on shared experts run in the same grouped FFN (all experts local)")
    ap.add_argument("--micro-batches", type=int, default=1, choices=[1, 2],
                    help="2: also time the two-micro-batch, two-stream schedule of the layer")
    ap.add_argument("--w-scales", default="", choices=["", "fp32", "pow2"],
                    help="fp8 weight block scales: any fp32 value or powers of two only "
                         "(default: the workload's own)")
    ap.add_argument("--eplb", action="store_true",
                    help="balanced expert placement from 8 calibration batches (EP-share workloads)")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# algorithmic work per stage (what the method must move / compute)
# ----------------------------------------------------------------------------
def stage_work(cfg, counts_local, tokens_with_local, K_slots=None):
    T, E, K, H, I = cfg.T, cfg.E, cfg.K if K_slots is None else K_slots, cfg.H, cfg.I
    R = int(counts_local.sum())
    touched = int((counts_local > 0).sum())
    sx, sa, sw, sy, so = (ESIZE[cfg.x_dtype], ESIZE[cfg.act_dtype], ESIZE[cfg.w_dtype],
                          ESIZE[cfg.y_dtype], ESIZE[cfg.out_dtype])
    nbH, nbI = -(-H // 128), -(-I // 128)
    fp8 = cfg.act_dtype == "fp8"
    sc_x = R * nbH * 4 if fp8 else 0
    sc_h = R * nbI * 4 if fp8 else 0
    sc_wgu = touched * 2 * I * nbH * 4 if cfg.w_dtype == "fp8" else 0
    sc_wd = touched * H * nbI * 4 if cfg.w_dtype == "fp8" else 0
    w = {
        "route": dict(bytes=T * E * 4 + T * K * 8, flops=0),
        "layout": dict(bytes=T * K * 4 * 3 + T * K * 4 + E * 4 * 2, flops=0),
        "dispatch": dict(bytes=tokens_with_local * H * sx + R * H * sa + sc_x, flops=0),
        "ffn_gate_up": dict(bytes=touched * 2 * I * H * sw + sc_wgu + R * H * sa + sc_x
                            + R * I * sa + sc_h, flops=4 * R * H * I),
        "ffn_down": dict(bytes=touched * H * I * sw + sc_wd + R * I * sa + sc_h + R * H * sy,
                         flops=2 * R * H * I),
        "combine": dict(bytes=R * H * sy + T * H * so + T * K * 8, flops=0),
    }
    return w, R, touched


def measured_traffic(workload: str):
    """Per-stage HBM bytes (read + write per launch) from the committed
    rocprofv3 PMC summary of this workload, calibrated against a plain copy
    kernel.  None when there is no summary or when any listed source file has
    changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    kv, stages = {}, {}
    for line in open(path):
        if line.startswith("stage ") and "=" in line:
            name, vals = line[6:].split("=", 1)
            r, w = (float(v) for v in vals.split())
            stages[name.strip()] = r + w
        elif " = " in line:
            k, v = line.split(" = ", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256()
    try:
        for f in kv["source_files"].split():
            with open(os.path.join(ROOT, f), "rb") as fh:
                sha.update(fh.read())
    except (KeyError, OSError):
        return None
    return stages if sha.hexdigest() == kv.get("source_sha256") else None


def measured_copy_gbs(dev, mib=1024, reps=5):
    """Achievable-bandwidth reference: GB/s (read + write) of torch's device
    copy of `mib` MiB, timed with events."""
    src = torch.empty(mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    gbs = 2 * src.numel() * 4 * reps / (t0.elapsed_time(t1) / 1e3) / 1e9
    del src, dst
    return gbs


def _group_loads(counts, G):
    c = np.asarray(counts, dtype=np.int64)
    return c.reshape(G, -1).sum(axis=1)


def eplb_placement(m, cfg, dev, batches=8):
    """Balanced placement of the experts over E / E_loc ranks from the
    activation counts of `batches` calibration batches, all counted by the
    library (route + layout on the GPU) and placed by moe_eplb_place."""
    G = cfg.E // cfg.E_loc
    if G * cfg.E_loc != cfg.E or cfg.e_begin % cfg.E_loc:
        raise SystemExit("--eplb needs a local range that is one of E / E_loc equal groups")
    lg = wl.gen_calibration_logits(cfg, 1000, batches=batches).to(dev)
    ids, _ = m.moe_route(lg, cfg.K)
    lay = m.moe_layout(ids, cfg.E, 0, cfg.E, ids.numel())
    counts = lay["counts"].cpu().numpy()
    phys = m.moe_eplb_place(counts, G).numpy()
    logical_of_phys = np.argsort(phys)
    return {"G": G, "phys": phys, "map": torch.from_numpy(phys.astype(np.int32)).to(dev),
            "local_logical": [int(e) for e in logical_of_phys[cfg.e_begin:cfg.e_end]],
            "calib_counts": counts}


def eplb_report(m, cfg, logits, placement, layer):
    """Per-rank loads of the measured batch with contiguous expert chunks and
    with the placement (counts from the library's layout of each routing)."""
    G = placement["G"]
    ids, _ = m.moe_route(logits, cfg.K)
    before = _group_loads(m.moe_layout(ids, cfg.E, 0, cfg.E, ids.numel())["counts"].cpu().numpy(), G)
    after = _group_loads(layer.counts.cpu().numpy(), G)

    def stats(gl):
        gl = gl.astype(np.float64)
        return {"loads": [int(v) for v in gl], "max_over_min": round(float(gl.max() / gl.min()), 4),
                "balancedness": round(float(gl.mean() / gl.max()), 4)}
    return {"ranks": G, "contiguous_chunks": stats(before), "balanced_placement": stats(after),
            "calibration": "8 batches of the workload's size, other tokens, same router and bias"}


def two_micro_batches(m, cfg, x, logits, wdict, layer, steps, warmup):
    """Time the two-micro-batch, two-stream schedule (same inputs, same
    per-token results: checked bit for bit against the single-batch run)."""
    from combine_grouped_gemm_amd.layer import MicroBatchedLayer
    ref = layer.forward(x, logits, wdict).clone()
    mb = MicroBatchedLayer(cfg.seg_rows, layer.E_routed, layer.K_routed, cfg.H, cfg.I, cfg.e_begin,
                           cfg.e_end, cfg.act_dtype, cfg.y_dtype, cfg.out_dtype, device=ref.device)
    oa, ob = mb.forward(x, logits, wdict)
    torch.cuda.synchronize()
    same = bool(torch.equal(torch.cat([oa, ob]), ref))
    for _ in range(warmup):
        mb.forward(x, logits, wdict)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        mb.forward(x, logits, wdict)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / (ms / 1e3), 1),
            "bitwise_equal_to_single_batch": same, "split": [mb.a.T, mb.b.T]}


def graph_replay(layer, x, logits, wdict, steps, warmup):
    """Capture one step (the six library calls) as a HIP graph and time
    `steps` back-to-back replays; returns ms per replayed step."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(x, logits, wdict)
        with torch.cuda.graph(g, stream=s):
            layer.forward(x, logits, wdict)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(layer.T / (ms / 1e3), 1),
            "steps": steps}


def roofline_of(work, ms, mfma_peak):
    t = ms / 1e3
    gbs = work["bytes"] / t / 1e9
    tfl = work["flops"] / t / 1e12
    hbm_floor = work["bytes"] / (HBM_PEAK_GBS * 1e9)
    mfma_floor = work["flops"] / (mfma_peak * 1e12) if work["flops"] else 0.0
    if mfma_floor > hbm_floor:
        return {"bound": "mfma", "achieved": round(tfl, 2), "peak": mfma_peak, "unit": "TFLOP/s",
                "frac": round(tfl / mfma_peak, 4)}
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ----------------------------------------------------------------------------
def cpu_baseline(cfg, x_cpu, logits_cpu, weights, budget_s):
    import oracle
    from oracle import numerics as nx
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))

    def wnp(j):
        d = weights.expert(j, "cpu")
        if cfg.w_dtype == "fp8":
            return tuple(nx.dequantize_fp8_blocks(d[k].float().numpy().astype(np.float64),
                                                  d[k + "_scale"].numpy()) for k in ("gate", "up", "down"))
        return tuple(d[k].float().numpy().astype(np.float64) for k in ("gate", "up", "down"))

    x = np.concatenate([s.float().numpy().astype(np.float64) for s in x_cpu])
    lg = logits_cpu.numpy()
    t0 = time.perf_counter()
    ids, gates = oracle.route(lg, cfg.K)
    lay = oracle.layout(ids, cfg.E, cfg.e_begin, cfg.e_end, cfg.cap)
    t_route_layout = time.perf_counter() - t0
    R = int(lay["offsets"][-1])
    off = lay["offsets"]
    touched = [j for j in range(cfg.E_loc) if off[j + 1] > off[j]]
    # dispatch + FFN + combine over a growing prefix of the touched experts
    done, t_ffn, rows_done = 0, 0.0, 0
    t_disp = 0.0
    for j in touched:
        a, b = int(off[j]), int(off[j + 1])
        W = wnp(j)                                      # weight fetch: not timed
        t1 = time.perf_counter()
        xd, xs = oracle.dispatch(x[lay["src_of"][a:b] // cfg.K], np.arange(b - a)[:, None], b - a,
                                 cfg.act_dtype)
        t2 = time.perf_counter()
        xv = nx.dequantize_fp8_blocks(xd, xs) if cfg.act_dtype == "fp8" else xd
        oracle.expert_ffn(xv, *W, cfg.act_dtype, cfg.y_dtype)
        t3 = time.perf_counter()
        t_disp += t2 - t1
        t_ffn += t3 - t2
        done += 1
        rows_done += b - a
        if t_route_layout + t_disp + t_ffn > budget_s:
            break
    scale = len(touched) / max(done, 1)
    # combine over all tokens with synthetic y of the right shape (cost is shape-bound)
    y = np.zeros((R, cfg.H))
    t4 = time.perf_counter()
    oracle.combine(y, lay["row_of"], gates, cfg.out_dtype)
    t_comb = time.perf_counter() - t4
    est = t_route_layout + (t_disp + t_ffn) * scale + t_comb
    extrapolated = done < len(touched)
    return {"value": round(cfg.T / est, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "extrapolated": extrapolated,
            "sample": (f"route+layout+combine on all {cfg.T} tokens; dispatch+FFN on {done} of "
                       f"{len(touched)} touched experts ({rows_done} of {R} rows)"
                       + (f", extrapolated linearly to all touched experts (x{scale:.2f})" if extrapolated
                          else ", no extrapolation")
                       + "; weight fetch to host untimed"),
            "measured_s": round(t_route_layout + t_disp + t_ffn + t_comb, 2),
            "toy_single_thread": toy_single_thread()}


def toy_single_thread(reps=5):
    """The oracle's whole toy layer (8 x 8 tokens, E=16, K=2, H=128, I=256,
    fp32) with its numerical libraries held to one thread: tokens/s, best of
    `reps` runs."""
    import oracle
    from threadpoolctl import threadpool_limits
    cfg = wl.CONFIGS["toy"]
    xs = wl.gen_x(cfg)
    x = np.concatenate([t.numpy().astype(np.float64) for t in xs])
    lg = wl.gen_logits(cfg, xs).numpy()
    W = wl.gen_expert_weights(cfg, "cpu")
    mats = [tuple(t[j].double().numpy() for t in (W.gate, W.up, W.down)) for j in range(cfg.E_loc)]
    best = float("inf")
    with threadpool_limits(limits=1):
        for _ in range(reps):
            t0 = time.perf_counter()
            oracle.layer(x, lg, cfg.K, cfg.E, cfg.e_begin, cfg.e_end, lambda j: mats[j],
                         cfg.act_dtype, cfg.y_dtype, cfg.out_dtype)
            best = min(best, time.perf_counter() - t0)
    return {"value": round(cfg.T / best, 1), "unit": "tokens/s", "cores": 1, "workload": "toy",
            "note": "whole toy layer, best of 5, one thread"}


def _act_bytes(cfg, R):
    """Bytes of one buffer set a step touches: inputs, routing and the
    activations of the R dispatched rows."""
    sx, sa, sy, so = (ESIZE[cfg.x_dtype], ESIZE[cfg.act_dtype], ESIZE[cfg.y_dtype], ESIZE[cfg.out_dtype])
    return cfg.T * cfg.H * (sx + so) + cfg.T * cfg.E * 4 + R * (cfg.H * sa + cfg.I * sa + cfg.H * sy)


def _time_steps(sets, stages_of, steps, warmup, stream):
    """warmup + steps steps, step s on buffer set s % len(sets); returns
    (wall ms per step, per-stage event ms lists, per-step event ms)."""
    nset = len(sets)
    for s in range(warmup):
        for _, run in stages_of[s % nset]:
            run()
    torch.cuda.synchronize()
    n_st = len(stages_of[0])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_st + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        for i, (_, run) in enumerate(stages_of[s % nset]):
            run()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = [n for n, _ in stages_of[0]]
    per = {n: [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)] for i, n in enumerate(names)}
    step_ms = [ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)]
    return wall * 1e3 / steps, per, step_ms


def _stage_report(per, work, mfma_peak, copy_gbs):
    rep = {}
    for name, times in per.items():
        ms = float(np.mean(times))
        t = ms / 1e3
        r = roofline_of(work[name], ms, mfma_peak)
        rep[name] = {"ms": round(ms, 4), "ms_median": round(float(np.median(times)), 4),
                     "ms_p10": round(float(np.percentile(times, 10)), 4),
                     "ms_p90": round(float(np.percentile(times, 90)), 4),
                     "GB_s": round(work[name]["bytes"] / t / 1e9, 1),
                     "TFLOP_s": round(work[name]["flops"] / t / 1e12, 2),
                     "hbm_frac": round(work[name]["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4),
                     "mfma_frac": round(work[name]["flops"] / t / 1e12 / mfma_peak, 4),
                     "copy_frac": round(work[name]["bytes"] / t / 1e9 / copy_gbs, 4),
                     "bytes": int(work[name]["bytes"]), "flops": int(work[name]["flops"]),
                     "bound": r["bound"]}
    return rep


def run_workload(m, cfg, a, dev, copy_gbs, headline):
    """Time one workload; returns its report (the full line for the headline,
    a compact object otherwise)."""
    print(f"[bench] workload {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    x_cpu = wl.gen_x(cfg)
    logits_cpu = wl.gen_logits(cfg, x_cpu)
    placement = None
    if headline and a.eplb:
        placement = eplb_placement(m, cfg, dev)
        W = wl.gen_expert_weights(cfg, device=dev, experts=placement["local_logical"])
    elif headline and a.shared_experts:
        if cfg.e_end != cfg.E:
            raise SystemExit("--shared-experts needs the local range to end at E")
        W = wl.gen_expert_weights(cfg, device=dev,
                                  experts=list(range(cfg.e_begin, cfg.E + a.shared_experts)))
    else:
        W = wl.gen_expert_weights(cfg, device=dev)
    wdict = W.as_dict()
    if not a.dense_weights:
        # once, before any timing, as a weight loader would: rows at the packed pitch
        for k in ("gate", "up", "down"):
            wdict[k] = m.moe_pack_weights(wdict[k])
        torch.cuda.synchronize()
    layout = a.layout if headline else "contiguous"
    n_shared = a.shared_experts if headline else 0

    def new_layer():
        L = m.MoELayer(cfg.seg_rows, cfg.E, cfg.K, cfg.H, cfg.I, cfg.e_begin, cfg.e_end,
                       cfg.act_dtype, cfg.y_dtype, cfg.out_dtype, device=dev, layout=layout,
                       cap_per_expert=(a.cap_per_expert or None) if headline else None,
                       n_shared=n_shared)
        if placement is not None:
            L.expert_map = placement["map"]
        return L

    layer = new_layer()
    x = [t.to(dev) for t in x_cpu]
    logits = logits_cpu.to(dev)

    # parity gate before timing: routing and layout must equal the oracle's
    layer.forward(x, logits, wdict)
    torch.cuda.synchronize()
    import oracle
    if n_shared:
        ids, _ = oracle.route_shared(logits_cpu.numpy(), cfg.K, n_shared)
    else:
        ids, _ = oracle.route(logits_cpu.numpy(), cfg.K)
    if placement is not None:
        ids = placement["phys"][ids]
    lay = oracle.layout(ids, layer.E, layer.e_begin, layer.e_end, layer.cap)
    ref_row_of = (oracle.layout_masked(ids, cfg.E, cfg.e_begin, cfg.e_end, layer.cap_e)["row_of"]
                  if layer.masked else lay["row_of"])
    if not (np.array_equal(layer.topk_ids.cpu().numpy(), ids)
            and np.array_equal(layer.row_of.cpu().numpy(), ref_row_of)):
        raise RuntimeError(f"parity gate failed on {cfg.name}: routing/layout differ from the oracle")
    counts_local = lay["counts"][layer.e_begin:layer.e_end]
    local = (ids >= layer.e_begin) & (ids < layer.e_end)
    work, R, touched = stage_work(cfg, counts_local, int(local.any(axis=1).sum()), layer.K)

    # buffer sets for the cold pass: the same inputs copied into independent
    # buffers (the copies give identical routing, so the algorithmic work is
    # the same on every set)
    per_set = _act_bytes(cfg, R)
    n_sets = 1 if a.cold_mb <= 0 else max(2, min(16, int(a.cold_mb * 2**20 // max(per_set, 1)) + 1))
    sets = [(layer, x, logits)]
    for _ in range(n_sets - 1):
        sets.append((new_layer(), [t.clone() for t in x], logits.clone()))
    stages_of = [L.stages(xs, lg, wdict) for (L, xs, lg) in sets]
    stream = torch.cuda.current_stream()
    mfma_peak = MFMA_PEAK_TFLOPS[cfg.act_dtype]

    print(f"[bench] {cfg.name}: timing {a.steps} cold steps over {n_sets} buffer sets",
          file=sys.stderr, flush=True)
    ms_cold, per_cold, step_cold = _time_steps(sets, stages_of, a.steps, a.warmup, stream)
    print(f"[bench] {cfg.name}: timing {a.steps} warm steps on one buffer set", file=sys.stderr, flush=True)
    ms_warm, per_warm, step_warm = _time_steps(sets[:1], stages_of[:1], a.steps, a.warmup, stream)
    cold = _stage_report(per_cold, work, mfma_peak, copy_gbs)
    warm = _stage_report(per_warm, work, mfma_peak, copy_gbs)
    dom = max(cold, key=lambda k: cold[k]["ms"])
    roof = roofline_of(work[dom], cold[dom]["ms"], mfma_peak)
    traffic = measured_traffic(cfg.name)
    roof.update({"kernel": dom, "traffic": (int(traffic[dom]) if traffic and dom in traffic else None),
                 "algorithmic_bytes": int(work[dom]["bytes"]), "algorithmic_flops": int(work[dom]["flops"]),
                 "hbm_frac": cold[dom]["hbm_frac"], "mfma_frac": cold[dom]["mfma_frac"]})
    ffn_ms = cold["ffn_gate_up"]["ms"] + cold["ffn_down"]["ms"]
    ffn_flops = work["ffn_gate_up"]["flops"] + work["ffn_down"]["flops"]
    ffn_bytes = work["ffn_gate_up"]["bytes"] + work["ffn_down"]["bytes"]
    grouped = {"ms": round(ffn_ms, 4), "TFLOP_s": round(ffn_flops / (ffn_ms / 1e3) / 1e12, 2),
               "mfma_frac": round(ffn_flops / (ffn_ms / 1e3) / 1e12 / mfma_peak, 4),
               "GB_s": round(ffn_bytes / (ffn_ms / 1e3) / 1e9, 1),
               "hbm_frac": round(ffn_bytes / (ffn_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    warm_brief = {"ms_per_step": round(ms_warm, 4),
                  "tokens_per_s": round(cfg.T / (ms_warm / 1e3), 1),
                  "stages": {k: {"ms": v["ms"], "GB_s": v["GB_s"], "hbm_frac": v["hbm_frac"]}
                             for k, v in warm.items()}}
    config = {"workload": cfg.name, "T": cfg.T, "E": cfg.E, "K": cfg.K, "H": cfg.H, "I": cfg.I,
              "local_experts": [cfg.e_begin, cfg.e_end], "segments": len(cfg.seg_rows),
              "rows": R, "experts_touched": touched,
              "buffer_sets": n_sets, "buffer_set_MB": round(per_set / 2**20, 1),
              "weights": "dense" if a.dense_weights else "packed",
              **({"weight_scales": cfg.w_scales} if cfg.w_dtype == "fp8" else {})}
    if not headline:
        out = {"value": round(cfg.T / (ms_cold / 1e3), 1), "unit": "tokens/s",
               "ms_per_step": round(ms_cold, 4), "dtype": cfg.act_dtype, "config": config,
               "roofline": roof, "grouped_ffn": grouped,
               "stages": {k: {"ms": v["ms"], "GB_s": v["GB_s"], "TFLOP_s": v["TFLOP_s"],
                              "hbm_frac": v["hbm_frac"], "mfma_frac": v["mfma_frac"]}
                          for k, v in cold.items()},
               "warm": warm_brief}
        return out, None
    res = {
        "metric": "MoE-layer tokens/s on 1 GPU",
        "value": round(cfg.T / (ms_cold / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms_cold, 4),
        "ms_per_step_events": round(float(np.mean(step_cold)), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.act_dtype, "data": "synthetic (seeded; random-init expert weights)",
        "config": config,
        "roofline": roof,
        "grouped_ffn": grouped,
        "stages": cold,
        "warm": warm_brief,
        "hbm_reference": {"copy_GB_s": round(copy_gbs, 1),
                          "note": "device-to-device copy of 1 GiB measured in this run (read + write bytes); "
                                  "copy_frac of a stage = its algorithmic GB/s / this"},
    }
    if layout == "masked":
        res["config"]["layout"] = {"kind": "masked", "cap_per_expert": layer.cap_e}
    if n_shared:
        res["config"]["shared_experts"] = n_shared
    if placement is not None:
        res["config"]["placement"] = "balanced (8 calibration batches)"
        res["eplb"] = eplb_report(m, cfg, logits, placement, layer)
    if a.graph:
        res["graph_replay"] = graph_replay(layer, x, logits, wdict, a.steps, a.warmup)
    if a.micro_batches == 2:
        res["two_micro_batches"] = two_micro_batches(m, cfg, x, logits, wdict, layer, a.steps, a.warmup)
    keep = (x_cpu, logits_cpu, W)
    del sets, stages_of
    return res, keep


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "libmoeep runs on one GPU only (no multi-GPU path); --gpus must be 1"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    import combine_grouped_gemm_amd as m
    m.lib()                                     # loud failure if the HIP library is missing
    cfg = wl.CONFIGS[a.workload]
    if a.w_scales:
        cfg = dataclasses.replace(cfg, w_scales=a.w_scales)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    copy_gbs = measured_copy_gbs(dev)
    try:
        res, keep = run_workload(m, cfg, a, dev, copy_gbs, headline=True)
    except RuntimeError as e:
        print(json.dumps({"error": str(e)}))
        sys.exit(1)
    if a.copy_calibration_mib:
        # one elementwise kernel that reads n*4 bytes and writes n*4 bytes
        n = a.copy_calibration_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        res["copy_calibration_bytes"] = {"read": n * 4, "write": n * 4}
        del src, dst
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        x_cpu, logits_cpu, W = keep
        res["cpu_baseline"] = cpu_baseline(cfg, x_cpu, logits_cpu, W, a.cpu_budget_s)
    del keep
    torch.cuda.empty_cache()
    if not a.no_others:
        others = {}
        for name in ("toy", "dsv3_decode", "ep8_share", "gptoss_fp8", "dsv3_prefill"):
            if name == cfg.name:
                continue
            try:
                others[name], _ = run_workload(m, wl.CONFIGS[name], a, dev, copy_gbs, headline=False)
            except Exception as e:  # a failing sub-workload must not hide the headline
                others[name] = {"error": f"{type(e).__name__}: {e}"}
            torch.cuda.empty_cache()
        res["other_workloads"] = others
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
