"""Benchmark of the MoE layer forward on one MI355X.

A step is one moe_forward call (route -> count-first dispatch -> expert FFN
-> combine) over one batch of synthetic, HBM-resident inputs.  The default
workload is the largest one-GPU shape, the skewed prefill: T = 8192 tokens,
hidden 7168, 256 experts, top-8, capacity 512, SwiGLU intermediate 2048,
bf16 with float32 accumulation, router logits N(0, 1) plus a Zipf(1.1)
per-expert bias (some experts overflow their capacity, others stay empty).
Every other workload shape is timed as a short sweep: the fp32 layer, the
prefill token buckets 256 / 2048 / 8192, decode with shared experts at 1 / 8
/ 32 tokens, the ReLU-square shapes at 1 / 8 / 16 rows (distinct and
shared routes), sigmoid routing, and the skewed layer with e4m3 weights.

Printed: one JSON line with tokens/s (whole job), us per layer, the stage
breakdown from HIP events recorded by the library on its stream inside the
timed region, the roofline of the dominant kernel, and the CPU oracle timed
on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
F32_PEAK_TFLOPS = 157.3      # MI355X fp32 (the float32 layer's GEMMs run on the vector ALUs)
DECODE_ROWS_PER_EXPERT = 12  # the library's switch to the slot-indexed decode GEMMs
FUSE_MAX_T, FUSE_MAX_Q, FUSE_MAX_E = 8, 256, 256   # routing inside the gate/up decode launch
ORACLE_FLOPS = 4.6e8         # the oracle's rate on one core (double, widening per element)
CPU_SAMPLE_S = 20.0          # target length of the CPU oracle sample
N_BANKS = 4                  # rotating x / logits banks
MIN_WARMUP_S = 0.2           # shortest warm-up of a sweep workload
SWEEP_MIN_TIMED_S = 0.02     # shortest plain timed region of a sweep workload


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="skewed_bf16")
    ap.add_argument("--sweep", default="tiny_fp32,prefill_T256,prefill_T2048,prefill_T8192,"
                    "decode_T1,decode_T8,decode_T32,relu2_distinct_R1,relu2_shared_R1,"
                    "relu2_distinct_R8,relu2_shared_R8,relu2_distinct_R16,relu2_shared_R16,"
                    "sigmoid_T2048,skewed_fp8",
                    help="comma-separated extra workloads timed briefly ('' = none)")
    ap.add_argument("--dispatch", default="prefill_T2048,prefill_T8192,skewed_bf16",
                    help="comma-separated workloads whose moe_route / moe_dispatch (with the "
                         "x_disp row copy) are timed on their own ('' = none)")
    ap.add_argument("--routing-modes", default="relu2_distinct_R1,relu2_shared_R1,relu2_distinct_R8,"
                    "relu2_shared_R8,relu2_distinct_R16,relu2_shared_R16",
                    help="workloads timed with internal routing and with the same routes "
                         "preselected ('' = none)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one device copy of this size first (counter calibration)")
    ap.add_argument("--protocols", type=int, default=1,
                    help="1: also time cold calls (median/p95) and a captured graph of calls")
    ap.add_argument("--cpu-tokens", type=int, default=-1,
                    help="tokens of the CPU oracle sample (0 = skip, -1 = sized to about "
                         "20 s of oracle work)")
    return ap.parse_args()


def stage_bytes_flops(cs, R, touched, ab, wb):
    """Algorithmic bytes and flops of each stage of moe_forward for a batch
    with R kept rows and `touched` non-empty experts.  The forward copies
    token rows into the expert-contiguous buffer only for float32 layers;
    bf16 layers place routes only (the expert GEMM reads x in place), so
    their scatter moves route metadata alone."""
    T, H, E, k, I = cs.T, cs.H, cs.E, cs.k, cs.I
    Q = T * k
    r_max = min(Q, E * cs.C)
    n_w = 2 * I if cs.act == 0 else I
    sc = 4 if wb == 1 else 0          # e4m3 per-row scales
    st = {
        "route": (T * E * 4 + Q * 8, 0),
        "count": (Q * 4 + Q * 8 + E * 8, 0),
        "scatter": ((T * H * ab + R * H * ab if ab == 4 else 0) + Q * 16 + r_max * 4, 0),
        "gemm1": (touched * n_w * (H * wb + sc) + R * H * ab + R * I * ab, 2 * R * H * n_w),
        "gemm2": (touched * H * (I * wb + sc) + R * I * ab + R * H * ab + R * 8, 2 * R * I * H),
        "shared": (0, 0),
        "combine": (R * H * ab + T * H * ab + Q * 4, 0),
    }
    if cs.n_shared:
        Is, S = cs.I_shared, cs.n_shared
        sh1 = (S * 2 * Is * H * 2 + T * H * ab + T * S * Is * ab, S * 2 * T * H * 2 * Is)
        sh2 = (S * Is * H * 2 + T * S * Is * ab + T * H * 4, S * 2 * T * H * Is)
        if decode_mode(cs):
            # the decode launches stream the shared experts' weights too: their
            # gate/up in the gate/up launch, their down projection in the other
            st["gemm1"] = tuple(a + b for a, b in zip(st["gemm1"], sh1))
            st["gemm2"] = tuple(a + b for a, b in zip(st["gemm2"], sh2))
        else:
            st["shared"] = tuple(a + b for a, b in zip(sh1, sh2))
    if fused_mode(cs):
        # routing and dispatch run inside the gate/up launch
        moved = [st.pop(k) for k in ("route", "count", "scatter")]
        st["gemm1"] = (st["gemm1"][0] + sum(m[0] for m in moved), st["gemm1"][1])
        st.update(route=(0, 0), count=(0, 0), scatter=(0, 0))
    return st


def decode_mode(cs):
    """The library runs the slot-indexed decode GEMMs (bf16 layers with at most
    12 routes per expert on average)."""
    return cs.act_fmt != 0 and cs.T * cs.k <= DECODE_ROWS_PER_EXPERT * cs.E


def fused_mode(cs):
    """The gate/up decode launch also routes and dispatches the batch."""
    return (decode_mode(cs) and 0 < cs.T <= FUSE_MAX_T and cs.T * cs.k <= FUSE_MAX_Q
            and cs.E <= FUSE_MAX_E and cs.w_fmt == 1)


def flops_peak_tflops(cs):
    """Matrix peak of the layer's GEMM arithmetic: bf16 MFMA (e4m3 weights are
    widened to bf16 in registers), or the fp32 vector peak for float32 layers."""
    return F32_PEAK_TFLOPS if cs.act_fmt == 0 else BF16_PEAK_TFLOPS


def run_workload(name, steps, warmup, with_events=True, protocols=False, min_warmup_s=0.0,
                 min_timed_s=0.0, graph=False):
    import torch
    import routing_dispatch_expert_amd as rde
    import synth

    dev = "cuda:0"
    cs = synth.case(name)
    base = synth.make_inputs(cs, dev)
    banks = []
    for b in range(N_BANKS):
        cb = synth.replace(cs, seed=cs.seed + 1000 * b)
        banks.append((synth.make_x(cb, dev), synth.make_logits(cb, dev)))
    p = rde.make_problem(cs.T, cs.H, cs.E, cs.k, cs.I, cs.C, cs.n_shared, cs.I_shared,
                         act_dtype=cs.act_fmt, w_dtype=cs.w_fmt, act=cs.act,
                         renormalize=cs.renormalize, score_func=cs.score_func,
                         route_scale=cs.route_scale)
    n = rde.moe_workspace_bytes(p)
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    rde.moe_workspace_init(ws)
    adt = torch.float32 if cs.act_fmt == synth.FMT_F32 else torch.bfloat16
    out = torch.empty((cs.T, cs.H), dtype=adt, device=dev)
    offsets = torch.empty(cs.E + 1, dtype=torch.int32, device=dev)
    n_ev = rde.MOE_N_STAGES
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    for row in evs:          # torch creates the HIP event on its first record
        for e in row:
            e.record()
    torch.cuda.synchronize()

    def step(i, ev=None):
        x, lg = banks[i % N_BANKS]
        meta = dict(offsets=offsets)
        if ev is not None:
            meta["stage_events"] = ev
        rde.moe_forward(p, x, lg, base.score_bias, None, None, base.w13, base.w2, base.s13, base.s2,
                        base.w13_sh, base.w2_sh, out, meta, ws)

    # `warmup` steps, continued until min_warmup_s has passed (the short sweep
    # workloads: a layer of a few tens of microseconds then also starts at full
    # clocks)
    tw = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - tw < min_warmup_s:
        step(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    n_warm = i
    # timed region 1: plain steps (the throughput figure), at least
    # min_timed_s of them at the warm-up's rate, so that the synchronisations
    # bracketing the region stay small against it
    n_plain = steps
    if min_timed_s > 0 and i > 0:
        per_step = (time.perf_counter() - tw) / i
        n_plain = max(steps, int(math.ceil(min_timed_s / per_step)))
    t0 = time.perf_counter()
    for i in range(n_plain):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # timed region 2: the same steps with the library recording an event at
    # every stage boundary on its stream (per-kernel durations; each event
    # adds a few microseconds, so this region is not the throughput figure)
    wall_ev = None
    if with_events:
        t0 = time.perf_counter()
        for i in range(steps):
            step(i, evs[i])
        torch.cuda.synchronize()
        wall_ev = time.perf_counter() - t0
    proto = measure_protocols(step, torch) if protocols else None
    graph_us = measure_graph(step, torch) if graph else None
    if rde.moe_error(ws) != 0:
        raise RuntimeError("malformed routes reported on synthetic inputs")
    stages = {}
    if with_events:
        for s in range(1, n_ev):
            d = [evs[i][s - 1].elapsed_time(evs[i][s]) * 1e3 for i in range(steps)]  # us
            stages[rde.STAGES[s]] = sum(d) / len(d)
    # kept rows / touched experts of the last step's batch (outside the timed region)
    off = offsets.cpu().tolist()
    R = off[-1]
    touched = sum(1 for e in range(cs.E) if off[e + 1] > off[e])
    ab = 4 if cs.act_fmt == synth.FMT_F32 else 2
    wb = {synth.FMT_F32: 4, synth.FMT_BF16: 2, synth.FMT_E4M3: 1}[cs.w_fmt]
    return dict(cs=cs, steps=steps, n_plain=n_plain, n_warm=n_warm, wall=wall, wall_ev=wall_ev,
                stages=stages, R=R,
                touched=touched, bf=stage_bytes_flops(cs, R, touched, ab, wb), base=base,
                protocols=proto, graph_us=graph_us)


def dispatch_bytes(cs, R):
    """Algorithmic bytes of moe_route and of moe_dispatch with the row copy:
    route reads the logits and writes ids and weights; dispatch reads the
    ids, writes counts, offsets, route_dst and row_src, reads every token
    row once and writes one copy per kept route."""
    import synth
    T, H, E, k = cs.T, cs.H, cs.E, cs.k
    ab = 4 if cs.act_fmt == synth.FMT_F32 else 2
    Q = T * k
    route = T * E * 4 + Q * 8
    disp = Q * 4 + E * 4 + (E + 1) * 4 + Q * 4 + cs.r_max * 4 + T * H * ab + R * H * ab
    return route, disp


def measure_dispatch(name, calls=50, min_warmup_s=MIN_WARMUP_S):
    """moe_route and moe_dispatch (x_disp rows written) called on their own,
    over four rotating input banks, each call timed with events on the
    stream it runs on: the count-first dispatch as a standalone data move."""
    import torch
    import routing_dispatch_expert_amd as rde
    import synth

    dev = "cuda:0"
    cs = synth.case(name)
    p = rde.make_problem(cs.T, cs.H, cs.E, cs.k, cs.I, cs.C, cs.n_shared, cs.I_shared,
                         act_dtype=cs.act_fmt, w_dtype=cs.w_fmt, act=cs.act,
                         renormalize=cs.renormalize, score_func=cs.score_func,
                         route_scale=cs.route_scale)
    ws = torch.empty(rde.moe_workspace_bytes(p), dtype=torch.uint8, device=dev)
    rde.moe_workspace_init(ws)
    adt = torch.float32 if cs.act_fmt == synth.FMT_F32 else torch.bfloat16
    banks = []
    for b in range(N_BANKS):
        cb = synth.replace(cs, seed=cs.seed + 1000 * b)
        banks.append(dict(x=synth.make_x(cb, dev), lg=synth.make_logits(cb, dev),
                          bias=synth.make_score_bias(cb, dev),
                          ids=torch.empty((cs.T, cs.k), dtype=torch.int32, device=dev),
                          w=torch.empty((cs.T, cs.k), dtype=torch.float32, device=dev)))
    counts = torch.empty(cs.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(cs.E + 1, dtype=torch.int32, device=dev)
    row_src = torch.empty(cs.r_max, dtype=torch.int32, device=dev)
    route_dst = torch.empty((cs.T, cs.k), dtype=torch.int32, device=dev)
    x_disp = torch.empty((cs.r_max, cs.H), dtype=adt, device=dev)

    def route(i):
        b = banks[i % N_BANKS]
        rde.moe_route(p, b["lg"], b["bias"], b["ids"], b["w"], ws)

    def disp(i):
        b = banks[i % N_BANKS]
        rde.moe_dispatch(p, b["x"], b["ids"], counts, offsets, row_src, route_dst, x_disp, ws)

    for i in range(N_BANKS):
        route(i)
    tw = time.perf_counter()
    i = 0
    while time.perf_counter() - tw < min_warmup_s:
        route(i)
        disp(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    out = {}
    for label, fn in (("route", route), ("dispatch", disp)):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
        for i in range(calls):
            ev[i].record()
            fn(i)
        ev[calls].record()
        torch.cuda.synchronize()
        d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(calls))
        out[label] = d[len(d) // 2]
    # the last call's realised kept rows (outside the timed region)
    R = int(offsets[-1].item())
    if rde.moe_error(ws) != 0:
        raise RuntimeError("malformed routes reported on synthetic inputs")
    rb, db = dispatch_bytes(cs, R)
    gbps = db / (out["dispatch"] * 1e-6) / 1e9
    return {"calls": "moe_dispatch: count + scan, then route placement and the x_disp row "
                     "copy; median of %d back-to-back calls" % calls,
            "T": cs.T, "H": cs.H, "E": cs.E, "k": cs.k, "kept_rows": R,
            "dispatch_us": round(out["dispatch"], 2), "dispatch_alg_bytes": db,
            "dispatch_GBps": round(gbps, 1), "dispatch_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "route_us": round(out["route"], 2), "route_alg_bytes": rb,
            "route_GBps": round(rb / (out["route"] * 1e-6) / 1e9, 1)}


def measure_routing_modes(name, steps=50, min_warmup_s=MIN_WARMUP_S):
    """moe_forward of one workload with internal routing (logits in) and with
    the same routes preselected (ids and weights in, taken from one internal
    call beforehand): plain steps over one input bank, wall time per call."""
    import torch
    import routing_dispatch_expert_amd as rde
    import synth

    dev = "cuda:0"
    cs = synth.case(name)
    inp = synth.make_inputs(cs, dev)
    p = rde.make_problem(cs.T, cs.H, cs.E, cs.k, cs.I, cs.C, cs.n_shared, cs.I_shared,
                         act_dtype=cs.act_fmt, w_dtype=cs.w_fmt, act=cs.act,
                         renormalize=cs.renormalize, score_func=cs.score_func,
                         route_scale=cs.route_scale)
    ws = torch.empty(rde.moe_workspace_bytes(p), dtype=torch.uint8, device=dev)
    rde.moe_workspace_init(ws)
    adt = torch.float32 if cs.act_fmt == synth.FMT_F32 else torch.bfloat16
    out = torch.empty((cs.T, cs.H), dtype=adt, device=dev)
    ids = torch.empty((cs.T, cs.k), dtype=torch.int32, device=dev)
    w = torch.empty((cs.T, cs.k), dtype=torch.float32, device=dev)
    rde.moe_forward(p, inp.x, inp.logits, inp.score_bias, None, None, inp.w13, inp.w2, inp.s13,
                    inp.s2, inp.w13_sh, inp.w2_sh, out, dict(ids=ids, w=w), ws)

    def internal():
        rde.moe_forward(p, inp.x, inp.logits, inp.score_bias, None, None, inp.w13, inp.w2, inp.s13,
                        inp.s2, inp.w13_sh, inp.w2_sh, out, None, ws)

    def preselected():
        rde.moe_forward(p, inp.x, None, None, ids, w, inp.w13, inp.w2, inp.s13, inp.s2,
                        inp.w13_sh, inp.w2_sh, out, None, ws)

    res = {}
    for label, fn in (("internal", internal), ("preselected", preselected)):
        tw = time.perf_counter()
        i = 0
        while time.perf_counter() - tw < min_warmup_s:
            fn()
            i += 1
            if i % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        res[label] = (time.perf_counter() - t0) / steps * 1e6
    if rde.moe_error(ws) != 0:
        raise RuntimeError("malformed routes reported on synthetic inputs")
    return {"internal_us": round(res["internal"], 2), "preselected_us": round(res["preselected"], 2),
            "ratio": round(res["internal"] / res["preselected"], 3)}


def measure_graph(step, torch, graph_calls=64, graph_replays=10):
    """us per call of graph_calls back-to-back calls, rotating over the input
    banks, captured once into a HIP graph and replayed: the host's launch
    cost is paid once per replay, not per call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(graph_calls):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(graph_replays):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / (graph_replays * graph_calls) * 1e6


def measure_protocols(step, torch, groups=15, calls=20, graph_calls=64, graph_replays=10):
    """Two further views of the same call.
    cold: a 1 GiB device write before every call evicts L2 and the 256 MB
          last-level cache, and the call alone is timed with events on the
          stream it runs on (groups x calls samples; median and p95).
    graph: graph_calls back-to-back calls, rotating over the input banks,
          captured once into a HIP graph and replayed (launch cost amortised)."""
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    e0 = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
    e1 = [torch.cuda.Event(enable_timing=True) for _ in range(calls)]
    cold = []
    for g in range(groups):
        for c in range(calls):
            flush.fill_((g * calls + c) & 0xFF)
            e0[c].record()
            step(c)
            e1[c].record()
        torch.cuda.synchronize()
        cold += [e0[c].elapsed_time(e1[c]) * 1e3 for c in range(calls)]
    del flush
    cold.sort()
    per_call = measure_graph(step, torch, graph_calls, graph_replays) * 1e-6
    return {"cold_us_median": round(cold[len(cold) // 2], 2),
            "cold_us_p95": round(cold[int(len(cold) * 0.95)], 2),
            "cold_samples": f"{groups} x {calls} calls, a 1 GiB device write before each",
            "graph_us_per_call": round(per_call * 1e6, 2),
            "graph_calls": f"{graph_calls} calls captured in one graph, {graph_replays} replays"}


def kernel_source_sha256() -> str:
    """sha256 over the library's kernel sources (file names and bytes, in
    name order); a committed counter summary applies only while it matches."""
    d = os.path.join(ROOT, "routing_dispatch_expert_amd", "csrc")
    h = hashlib.sha256()
    for n in sorted(os.listdir(d)):
        if n.endswith((".hip", ".h")):
            h.update(n.encode())
            with open(os.path.join(d, n), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def counted_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` (FETCH_SIZE + WRITE_SIZE, each scaled by
    a plain copy's reading) from the committed counter summary of `workload`;
    None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"moe_forward_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        vals = dict(m.groups() for m in re.finditer(r"^([\w\[\]]+)=(\S+)$", f.read(), re.M))
    if vals.get("source_sha256") != kernel_source_sha256() or vals.get("workload") != workload:
        return None
    v = vals.get(f"traffic_bytes[{stage}]")
    return int(v) if v is not None else None


def dominant_gemm(res):
    """The longer of the two expert GEMMs: they carry the layer's weight bytes
    and flops (the other stages are a few microseconds, within event noise on
    small batches)."""
    return max(("gemm1", "gemm2"), key=lambda s: res["stages"][s])


def roofline_of(res, stage):
    us = res["stages"][stage]
    byts, flops = res["bf"][stage]
    fpk = flops_peak_tflops(res["cs"])
    t_hbm = byts / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (fpk * 1e12)
    if t_mfma > t_hbm:
        ach = flops / (us * 1e-6) / 1e12
        return {"bound": "mfma" if fpk == BF16_PEAK_TFLOPS else "alu", "achieved": round(ach, 1),
                "peak": fpk, "unit": "TFLOP/s", "frac": round(ach / fpk, 4),
                "traffic": counted_traffic(res["cs"].name, stage),
                "kernel": stage, "us": round(us, 2), "alg_flops": flops, "alg_bytes": byts}
    ach = byts / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBPS, 4),
            "traffic": counted_traffic(res["cs"].name, stage), "kernel": stage,
            "us": round(us, 2), "alg_bytes": byts, "alg_flops": flops}


def layer_work(cs, R, touched):
    """Algorithmic bytes and flops of the whole layer, counted as the method
    moves them: the non-empty experts' weights (and the shared experts'), the
    logits and route metadata, x read once, the expert-contiguous row copy and
    the intermediate h each written and read once, and out written."""
    T, H, E, k, I = cs.T, cs.H, cs.E, cs.k, cs.I
    ab = 4 if cs.act_fmt == 0 else 2
    wb = {0: 4, 1: 2, 2: 1}[cs.w_fmt]
    n_w = 2 * I if cs.act == 0 else I
    sc = 4 * (n_w + H) if cs.w_fmt == 2 else 0
    byts = touched * ((n_w + I) * H * wb + sc)
    byts += T * E * 4 + T * k * 16 + T * H * ab + 2 * R * H * ab + 2 * R * I * ab + T * H * ab
    flops = 2 * R * H * (n_w + I) + 2 * R * H
    if cs.n_shared:
        Is, S = cs.I_shared, cs.n_shared
        byts += S * 3 * Is * H * 2
        flops += S * 2 * T * H * 3 * Is
    return byts, flops


def layer_roofline(res, ceiling_gbps=None):
    """t_roofline / t_measured for the whole layer, t_roofline = max(bytes /
    HBM peak, flops / matrix peak); `frac_measured` takes the measured HBM
    ceiling of the same run (the faster of a device copy and a read stream)
    in place of the HBM peak."""
    byts, flops = layer_work(res["cs"], res["R"], res["touched"])
    fpk = flops_peak_tflops(res["cs"])
    t_meas = res["wall"] / res.get("n_plain", res["steps"])
    t_h, t_m = byts / (HBM_PEAK_GBPS * 1e9), flops / (fpk * 1e12)
    out = {"alg_bytes": byts, "alg_flops": flops, "t_hbm_us": round(t_h * 1e6, 2),
           "t_mfma_us": round(t_m * 1e6, 2),
           "bound": ("mfma" if fpk == BF16_PEAK_TFLOPS else "alu") if t_m > t_h else "hbm",
           "t_roofline_us": round(max(t_h, t_m) * 1e6, 2),
           "frac": round(max(t_h, t_m) / t_meas, 4)}
    if ceiling_gbps:
        t_hc = byts / (ceiling_gbps * 1e9)
        out["frac_measured"] = round(max(t_hc, t_m) / t_meas, 4)
    return out


def measure_copy_gbps(torch, mib=1024, reps=5):
    """Device-to-device copy of `mib` MiB: bytes read + written per second."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return round(2 * n / sec / 1e9, 1)


def measure_read_gbps(torch, mib=2048, reps=5):
    """A read stream: row sums of a `mib` MiB float32 tensor of 4096-float
    rows (every byte read once per call; one float written per 16 KiB row):
    bytes read per second.  Of the torch reductions and products tried on
    MI355X this one streams fastest (a whole-tensor sum is slower than a
    device copy)."""
    n = (mib << 20) // 4
    src = torch.ones((n // 4096, 4096), dtype=torch.float32, device="cuda:0")
    for _ in range(2):
        src.sum(dim=1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        src.sum(dim=1)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src
    return round(4 * n / sec / 1e9, 1)


def summary(res, ceiling_gbps=None):
    cs, st, bf = res["cs"], res["stages"], res["bf"]
    disp_us = st["count"] + st["scatter"]
    disp_b = bf["count"][0] + bf["scatter"][0]
    g_us = st["gemm1"] + st["gemm2"]
    g_fl = bf["gemm1"][1] + bf["gemm2"][1]
    return {
        "us_per_layer": round(res["wall"] / res.get("n_plain", res["steps"]) * 1e6, 2),
        "sum_of_stage_us": round(sum(st.values()), 2),
        "dispatch_us": round(disp_us, 2),
        "dispatch_bytes": disp_b,
        "gemm_mfma_pct": round(100 * g_fl / (g_us * 1e-6) / (flops_peak_tflops(cs) * 1e12), 2),
        "gemm_hbm_GBps": round((bf["gemm1"][0] + bf["gemm2"][0]) / (g_us * 1e-6) / 1e9, 1),
        "kept_rows": res["R"], "experts_touched": res["touched"],
        "stages_us": {k: round(v, 2) for k, v in st.items()},
        "ms_per_step_with_stage_events": round(res["wall_ev"] / res["steps"] * 1e3, 4)
        if res.get("wall_ev") else None,
        "layer_roofline": layer_roofline(res, ceiling_gbps),
    }


def cpu_sample_tokens(cs):
    """Tokens of the CPU oracle sample: about CPU_SAMPLE_S seconds of oracle
    work at its single-core rate (every route of the sample is assumed kept)."""
    n_w = 2 * cs.I if cs.act == 0 else cs.I
    per_token = cs.k * 2 * cs.H * (n_w + cs.I)
    if cs.n_shared:
        per_token += cs.n_shared * 2 * cs.H * 3 * cs.I_shared
    return int(max(1, min(cs.T, round(CPU_SAMPLE_S * ORACLE_FLOPS / per_token))))


def cpu_baseline(res, n_tokens):
    """The oracle as it stands, single-threaded, on the first n_tokens tokens
    of the same workload (same weights, capacity and expert count).  Only the
    experts those tokens route to are copied to the host.  Besides the
    sample's own rate, the whole layer is extrapolated from its time per kept
    route (the full batch keeps res['R'] routes; on the skewed workload most
    routes are dropped by capacity, which a short sample of early tokens does
    not see)."""
    import numpy as np
    import oracle
    import synth

    cs = res["cs"]
    sub = synth.replace(cs, T=n_tokens)
    base = res["base"]
    conv = lambda t: None if t is None else oracle.from_torch(t)
    x = conv(base.x[:n_tokens])
    lg = conv(base.logits[:n_tokens])
    bias = conv(base.score_bias)
    ids, _ = oracle.route(lg, cs.k, cs.renormalize, cs.score_func, bias, cs.route_scale)
    touched = sorted(set(ids.ravel().tolist()))

    def host_weights(t):
        if t is None:
            return None
        h = np.zeros(tuple(t.shape), dtype=conv(t[:1]).dtype)   # untouched experts stay zero pages
        for e in touched:
            h[e] = conv(t[e])
        return h

    w13, w2, s13, s2 = (host_weights(t) for t in (base.w13, base.w2, base.s13, base.s2))
    r = oracle.forward(sub, x, lg, w13, w2, s13, s2, conv(base.w13_sh), conv(base.w2_sh),
                       score_bias=bias)
    sec = r["seconds"]
    kept = int(r["offsets"][-1])
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:
        host_cores = os.cpu_count()
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    per_route = sec / max(kept, 1)
    full_s = per_route * res["R"] if kept else sec / n_tokens * cs.T
    return {"value": round(n_tokens / sec, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host_cores": host_cores, "cpu_model": model,
            "sample": f"first {n_tokens} of {cs.T} tokens of {cs.name} ({kept} kept routes): "
                      f"routing, count-first dispatch, expert FFN and combine for them, "
                      f"{sec:.1f} s on one core",
            "us_per_kept_route": round(per_route * 1e6, 1),
            "us_per_layer_extrapolated": round(full_s * 1e6, 1),
            "tokens_per_s_extrapolated": round(cs.T / full_s, 3),
            "extrapolation": f"time per kept route x the {res['R']} kept routes of the full batch"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              f"multi-GPU path: see the sharding design notes.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: {n} bytes", file=sys.stderr, flush=True)
        del src, dst
    print(f"[bench] workload {args.workload}: warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    # at least MIN_WARMUP_S of warm-up steps (more than --warmup when those
    # take less): the GPU reaches its steady clocks before the timed region
    res = run_workload(args.workload, args.steps, args.warmup, protocols=bool(args.protocols),
                       min_warmup_s=MIN_WARMUP_S)
    copy_gbps = measure_copy_gbps(torch) if args.protocols else None
    read_gbps = measure_read_gbps(torch) if args.protocols else None
    ceiling = max(copy_gbps, read_gbps) if args.protocols else None
    cs = res["cs"]
    ms = res["wall"] / res["n_plain"] * 1e3
    summ = summary(res, ceiling)
    dom = dominant_gemm(res)
    line = {
        "metric": "MoE layer tokens/s + us/layer; dispatch HBM GB/s, grouped-GEMM MFMA % of peak",
        "value": round(cs.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "warmup_steps_run": res["n_warm"],
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cs.act_fmt == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": cs.name, "T": cs.T, "H": cs.H, "E": cs.E, "k": cs.k, "I": cs.I,
                   "C": cs.C, "act": "swiglu" if cs.act == 0 else "relu2",
                   "weights": {0: "f32", 1: "bf16", 2: "e4m3"}[cs.w_fmt],
                   "n_shared": cs.n_shared, "parallelism": "none (1 GPU)"},
        **summ,
        "roofline": roofline_of(res, dom),
        "copy_GBps": copy_gbps,
        "read_GBps": read_gbps,
        "hbm_ceiling_GBps": ceiling,
    }
    if res.get("protocols"):
        pr = dict(res["protocols"])
        pr["graph_tokens_per_s"] = round(cs.T / (pr["graph_us_per_call"] * 1e-6), 1)
        line["protocols"] = pr
    print(f"[bench] {cs.name}: {ms*1e3:.1f} us/step, stages {summ['stages_us']}",
          file=sys.stderr, flush=True)
    n_cpu = cpu_sample_tokens(cs) if args.cpu_tokens < 0 else args.cpu_tokens
    if n_cpu > 0:
        print(f"[bench] cpu baseline: oracle on {n_cpu} tokens", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(res, n_cpu)
    del res["base"]
    sweep = {}
    for name in [s for s in args.sweep.split(",") if s]:
        print(f"[bench] sweep {name}", file=sys.stderr, flush=True)
        r2 = run_workload(name, max(5, args.steps // 3), 10, min_warmup_s=MIN_WARMUP_S,
                          min_timed_s=SWEEP_MIN_TIMED_S, graph=True)
        ms2 = r2["wall"] / r2["n_plain"] * 1e3
        sw = summary(r2, ceiling)
        sw["tokens_per_s"] = round(r2["cs"].T / (ms2 * 1e-3), 1)
        sw["ms_per_step"] = round(ms2, 4)
        sw["steps"] = r2["n_plain"]
        sw["graph_us_per_call"] = round(r2["graph_us"], 2)
        d2 = dominant_gemm(r2)
        sw["roofline"] = roofline_of(r2, d2)
        sweep[name] = sw
        del r2
        torch.cuda.empty_cache()
    if sweep:
        line["sweep"] = sweep
    modes = {}
    for name in [s for s in args.routing_modes.split(",") if s]:
        print(f"[bench] routing modes {name}", file=sys.stderr, flush=True)
        modes[name] = measure_routing_modes(name)
        torch.cuda.empty_cache()
    if modes:
        line["routing_modes"] = modes
    disp = {}
    for name in [s for s in args.dispatch.split(",") if s]:
        print(f"[bench] dispatch {name}", file=sys.stderr, flush=True)
        disp[name] = measure_dispatch(name)
        torch.cuda.empty_cache()
    if disp:
        line["dispatch"] = disp
        main_d = disp.get(cs.name)
        if main_d is not None:
            line["dispatch_GBps"] = main_d["dispatch_GBps"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
