"""Throughput of the ternary projection's forward + backward on one MI355X.

One step = for every projection of one layer of the workload: materialize
(q -> 2-bit tern), forward (Y), input gradient (dX) and weight-side gradients
(gq, sgrad), all through the C ABI on one stream, inputs already resident in
HBM.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large] [--launch eager|graph]

By default a step is the layer calls (tern_layer_*: one call per product for
all projections; --api projection uses the single-projection calls), recorded
once as a HIP graph (tern_graph_*) with the dW call (and, for small products,
the dX call) on branches of their own (--streams), and its replays are timed
(--launch eager times the calls themselves); the per-part times always come
from eager calls, timed with events between them.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
COPY_BYTES = 1 << 30  # calibration copy size


def kernel_src_hash() -> str:
    """Key of the stored traffic counters: the kernels and the planner's code."""
    from ternary_weight_linear_tern_amd.rocprof_summary import kernel_code_hash
    return kernel_code_hash()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large", choices=["rwkv_small", "mid", "large", "largest"])
    ap.add_argument("--launch", default="graph", choices=["eager", "graph"],
                    help="graph (default): time replays of one recorded step; eager: time the calls")
    ap.add_argument("--streams", default="auto", choices=["auto", "1", "2", "3", "p3"],
                    help="graph branches of the recorded step: 1 = one chain; 2 = dW on its own branch; 3 = dX "
                         "and dW each on their own branch (after the materialize); p3 (single-projection "
                         "calls only) = whole projections dealt over three branches; auto: layer calls take 3 "
                         "when the forward or dX product of the layer has fewer 512 x 128 tiles than the GPU "
                         "has compute units (small products, whose latencies then overlap), else 1 (every "
                         "product fills the chip on its own, and a concurrent one only competes for its L2 "
                         "and clock); single calls take p3 when some projection's forward or dX has fewer "
                         "tiles than compute units, else 2")
    ap.add_argument("--api", default="layer", choices=["layer", "projection"],
                    help="layer (default): one call per product for all projections (tern_layer_*); "
                         "projection: the single-projection calls, one per projection and product")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=3072, help="oracle sample: token rows per projection")
    ap.add_argument("--cpu-cols", type=int, default=768, help="oracle sample: output columns per projection")
    ap.add_argument("--cpu-1t-div", type=int, default=16,
                    help="the 1-thread oracle runs on 1/N of the all-thread sample's rows and columns")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the board-power window (the step repeated for about 1.5 s after the timed region "
                         "while the board's power sensor is sampled)")
    ap.add_argument("--no-vendor-gemm", action="store_true",
                    help="skip the context line: dense bf16 torch.mm (hipBLASLt) on the same three products")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, copy a 1 GiB buffer 3 times (known bytes, for scaling "
                         "HBM traffic counters)")
    ap.add_argument("--extras", action="store_true",
                    help="instead of the step: per-call times of the accumulating backward, the q/k/v "
                         "group, the health panel and the scale step on the workload's shapes (eager, one "
                         "JSON line)")
    return ap.parse_args()


def extras(a):
    """Per-call times of the entry points beyond the step, on the workload's
    projections (eager calls, events on the current stream, median of a few
    timed repetitions): dX and dW plain against accumulating, the fused q/k/v
    group against three separate projections, the gather that builds it, the
    health panel with churn, and the scale's AdamW step.  HBM-bound calls are
    also given against their algorithmic bytes and the 8 TB/s peak."""
    import statistics

    import numpy as np
    import torch

    import synth
    import ternary_weight_linear_tern_amd as tl

    w = synth.WORKLOADS[a.workload]
    torch.cuda.set_device(0)

    def to_dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    projs = []
    for i, (name, n_in, n_out) in enumerate(w.projs):
        p = synth.workload_inputs(w, i)
        d = dict(name=name, n_in=n_in, n_out=n_out, X=to_dev(p.X), dY=to_dev(p.dY), q=to_dev(p.q),
                 scale=to_dev(p.scale), theta=p.theta)
        d["packed"] = tl.empty_packed(n_in, n_out)
        d["prev"] = tl.empty_packed(n_in, n_out)
        d["dX"] = torch.empty((w.T, n_in), device="cuda")
        d["Y"] = torch.empty((w.T, n_out), device="cuda")
        d["gq"] = torch.zeros((n_in, n_out), device="cuda")
        d["sgrad"] = torch.zeros((n_out,), device="cuda")
        d["ws"] = tl.empty_workspace(w.T, n_in, n_out)
        d["ws_acc"] = tl.empty_workspace(w.T, n_in, n_out, acc=True)
        d["m"] = torch.zeros((n_out,), device="cuda")
        d["v"] = torch.zeros((n_out,), device="cuda")
        tl.tern_materialize(d["q"], d["theta"], d["packed"])
        tl.tern_materialize(torch.roll(d["q"], 1, 1).contiguous(), d["theta"], d["prev"])
        projs.append(d)
    torch.cuda.synchronize()
    print(f"# extras: inputs ready, workload {w.name}", file=sys.stderr, flush=True)

    def timed(fn, reps=8, warm=2):
        for _ in range(warm):
            fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts)   # ms

    out = {}
    flops = sum(2.0 * w.T * d["n_in"] * d["n_out"] for d in projs)
    dx = timed(lambda: [tl.tern_linear_bwd_dx(d["dY"], d["packed"], d["scale"], d["dX"]) for d in projs])
    dxa = timed(lambda: [tl.tern_linear_bwd_dx_acc(d["dY"], d["packed"], d["scale"], d["dX"]) for d in projs])
    dw = timed(lambda: [tl.tern_linear_bwd_dw(d["X"], d["dY"], d["packed"], d["scale"], d["gq"], d["sgrad"],
                                              d["ws"]) for d in projs])
    dwa = timed(lambda: [tl.tern_linear_bwd_dw_acc(d["X"], d["dY"], d["packed"], d["scale"], d["gq"], d["sgrad"],
                                                   d["ws_acc"], 0.5) for d in projs])
    for k, ms in (("bwd_dx", dx), ("bwd_dx_acc", dxa), ("bwd_dw", dw), ("bwd_dw_acc", dwa)):
        out[k] = {"ms_per_step": round(ms, 4), "tflops": round(flops / ms / 1e9, 1),
                  "mfma_frac": round(flops / ms / 1e9 / PEAK_TFLOPS["bf16"], 4)}

    # health panel over every projection, churn against a previous handle:
    # q (1 B), the previous canonical codes (1/4 B) per weight, scale (4 B) per column
    panel = tl.empty_panel()

    def panel_pass():
        tl.tern_panel_reset(panel)
        for d in projs:
            tl.tern_panel_add(d["q"], d["theta"], d["scale"], panel, prev_packed=d["prev"])
    ms = timed(panel_pass)
    nb = sum(d["n_in"] * d["n_out"] * 1.25 + 4 * d["n_out"] for d in projs)
    out["panel"] = {"ms_per_step": round(ms, 4), "bytes": nb, "gbs": round(nb / ms / 1e6, 1),
                    "hbm_frac": round(nb / ms / 1e6 / PEAK_HBM_GBS, 4)}

    # scale step: sgrad, scale, m, v read and scale, m, v written (28 B per column)
    stp = [1]

    def adamw_pass():
        stp[0] += 1
        for d in projs:
            tl.tern_scale_adamw(d["sgrad"], d["scale"], d["m"], d["v"], stp[0], 1e-3, 1e-3)
    ms = timed(adamw_pass)
    ncols = sum(d["n_out"] for d in projs)
    out["scale_adamw"] = {"ms_per_step": round(ms, 4), "us_per_call": round(1000 * ms / len(projs), 2),
                          "bytes": 28 * ncols}

    # q/k/v as one group: the three square projections of the block that read one input
    mem = [d for d in projs if d["n_in"] == d["n_out"]][:3]
    if len(mem) == 3:
        n_in = mem[0]["n_in"]
        tot = sum(d["n_out"] for d in mem)
        qg = torch.empty((n_in, tot), dtype=torch.int8, device="cuda")
        sg = torch.empty((tot,), device="cuda")
        ms = timed(lambda: tl.tern_group_gather([d["q"] for d in mem], [d["scale"] for d in mem], qg, sg))
        nb = 2.0 * (n_in * tot + 4 * tot)
        out["group_gather"] = {"ms": round(ms, 4), "bytes": nb, "gbs": round(nb / ms / 1e6, 1),
                               "hbm_frac": round(nb / ms / 1e6 / PEAK_HBM_GBS, 4)}
        pk = tl.empty_packed(n_in, tot)
        tl.tern_materialize(qg, mem[0]["theta"], pk)
        X = mem[0]["X"]
        dYg = torch.cat([d["dY"] for d in mem], dim=1).contiguous()
        Yg = torch.empty((w.T, tot), device="cuda")
        dXg = torch.empty((w.T, n_in), device="cuda")
        gqg = torch.empty((n_in, tot), device="cuda")
        sgg = torch.empty((tot,), device="cuda")
        wsg = tl.empty_workspace(w.T, n_in, tot)
        gf = timed(lambda: tl.tern_linear_fwd(X, pk, sg, Yg))
        sf = timed(lambda: [tl.tern_linear_fwd(X, d["packed"], d["scale"], d["Y"]) for d in mem])
        gb = timed(lambda: tl.tern_linear_bwd(X, dYg, pk, sg, dXg, gqg, sgg, wsg))

        def sep_bwd():
            for j, d in enumerate(mem):
                (tl.tern_linear_bwd_dx if j == 0 else tl.tern_linear_bwd_dx_acc)(d["dY"], d["packed"], d["scale"],
                                                                                 dXg)
                tl.tern_linear_bwd_dw(X, d["dY"], d["packed"], d["scale"], d["gq"], d["sgrad"], d["ws"])
        sb = timed(sep_bwd)
        out["qkv_group"] = {"fwd_ms": round(gf, 4), "fwd_separate_ms": round(sf, 4), "bwd_ms": round(gb, 4),
                            "bwd_separate_ms": round(sb, 4)}
    torch.cuda.synchronize()
    print(json.dumps({"metric": "per-call times of the entry points beyond the step", "workload": w.name,
                      "T": w.T, "projections": [[d["name"], d["n_in"], d["n_out"]] for d in projs],
                      "launch": "eager", "entries": out}), flush=True)


def ready_events(events, stream):
    """Record every timing event once before a timed region: torch creates
    the device event at its first record, and a creation that stalls the host
    inside the region would count as GPU time of the part being enqueued."""
    import torch
    for e in events:
        e.record(stream)
    torch.cuda.synchronize()


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py runs on exactly one GPU; --gpus {a.gpus} is not supported "
              "(the library has no multi-GPU path; sharding is described, not built)", file=sys.stderr, flush=True)
        sys.exit(2)

    if a.extras:
        extras(a)
        return

    import numpy as np
    import torch

    import synth
    import ternary_weight_linear_tern_amd as tl

    w = synth.WORKLOADS[a.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def to_dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    t0 = time.time()
    projs = []
    for i, (name, n_in, n_out) in enumerate(w.projs):
        p = synth.workload_inputs(w, i)
        d = dict(name=name, n_in=n_in, n_out=n_out, X=to_dev(p.X), dY=to_dev(p.dY), q=to_dev(p.q),
                 scale=to_dev(p.scale), theta=p.theta)
        d["packed"] = tl.empty_packed(n_in, n_out)
        d["Y"] = torch.empty((w.T, n_out), dtype=torch.float32, device=dev)
        d["dX"] = torch.empty((w.T, n_in), dtype=torch.float32, device=dev)
        d["gq"] = torch.empty((n_in, n_out), dtype=torch.float32, device=dev)
        d["sgrad"] = torch.empty((n_out,), dtype=torch.float32, device=dev)
        d["ws"] = tl.empty_workspace(w.T, n_in, n_out)
        d["host"] = p if not a.no_cpu_baseline else None
        projs.append(d)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f}s: workload {w.name} T={w.T} "
          f"projections {[(d['name'], d['n_in'], d['n_out']) for d in projs]}", file=sys.stderr, flush=True)

    PARTS = ("materialize", "fwd", "bwd_dx", "bwd_dw")
    layer = a.api == "layer"
    layer_ws = tl.empty_layer_workspace([(d["n_in"], d["n_out"]) for d in projs], w.T) if layer else None
    theta = projs[0]["theta"]

    def step_layer(evs=None, stream=stream):
        # one call per product for all projections; the events of a step sit
        # in slot 0 (the parts of the whole layer)
        if evs is not None:
            evs[0][0].record(stream)
        tl.tern_layer_materialize(projs, theta, stream)
        if evs is not None:
            evs[0][1].record(stream)
        tl.tern_layer_fwd(projs, stream)
        if evs is not None:
            evs[0][2].record(stream)
        tl.tern_layer_bwd_dx(projs, stream)
        if evs is not None:
            evs[0][3].record(stream)
        tl.tern_layer_bwd_dw(projs, layer_ws, stream)
        if evs is not None:
            evs[0][4].record(stream)

    def step(evs=None, stream=stream):
        if layer:
            return step_layer(evs, stream)
        for j, d in enumerate(projs):
            if evs is not None:
                evs[j][0].record(stream)
            tl.tern_materialize(d["q"], d["theta"], d["packed"], stream)
            if evs is not None:
                evs[j][1].record(stream)
            tl.tern_linear_fwd(d["X"], d["packed"], d["scale"], d["Y"], stream)
            if evs is not None:
                evs[j][2].record(stream)
            tl.tern_linear_bwd_dx(d["dY"], d["packed"], d["scale"], d["dX"], stream=stream)
            if evs is not None:
                evs[j][3].record(stream)
            tl.tern_linear_bwd_dw(d["X"], d["dY"], d["packed"], d["scale"], d["gq"], d["sgrad"], d["ws"],
                                  stream)
            if evs is not None:
                evs[j][4].record(stream)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: events on the stream every kernel is launched on
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in projs] for _ in range(a.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ready_events([e for k in evs for j in k for e in j] + [start, end], stream)

    def eager_region():
        start.record(stream)
        for k in range(a.steps):
            step(evs[k])
        end.record(stream)
        torch.cuda.synchronize()

    # The region runs twice and the second is kept: the first launches of a
    # run that queues this many dispatches and events ahead of the GPU have
    # stalled the host for 30-40 ms once (inside the second step, whatever
    # the workload), which is runtime set-up, not the kernels' time.
    eager_region()
    eager_region()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / a.steps

    def record_dag(streams):
        """The step as a DAG: every projection's forward, dX and dW depend only
        on its materialize.  Branch streams join the recording through events
        recorded on the first stream and rejoin it at the end."""
        s0 = streams[0]
        sdx, sdw = streams[1 if len(streams) == 3 else 0], streams[-1]

        def fork(src, dst):
            e = torch.cuda.Event()
            e.record(src)
            dst.wait_event(e)

        for sx in streams[1:]:
            fork(s0, sx)
        for d in projs:
            tl.tern_materialize(d["q"], d["theta"], d["packed"], s0)
            for sx in streams[1:]:
                fork(s0, sx)
            tl.tern_linear_fwd(d["X"], d["packed"], d["scale"], d["Y"], s0)
            tl.tern_linear_bwd_dx(d["dY"], d["packed"], d["scale"], d["dX"], stream=sdx)
            tl.tern_linear_bwd_dw(d["X"], d["dY"], d["packed"], d["scale"], d["gq"], d["sgrad"], d["ws"], sdw)
        for sx in streams[1:]:
            fork(sx, s0)

    def record_layer(streams):
        """The layer step as a DAG: materialize, then the forward, dX and dW
        calls, each on its own branch when there are three streams."""
        s0 = streams[0]
        # 2 streams: forward and dX on the first, dW on the second; 3: one each
        sdx = streams[1] if len(streams) == 3 else s0
        sdw = streams[-1]

        def fork(src, dst):
            e = torch.cuda.Event()
            e.record(src)
            dst.wait_event(e)

        tl.tern_layer_materialize(projs, theta, s0)
        for sx in streams[1:]:
            fork(s0, sx)
        tl.tern_layer_fwd(projs, s0)
        tl.tern_layer_bwd_dx(projs, sdx)
        tl.tern_layer_bwd_dw(projs, layer_ws, sdw)
        for sx in streams[1:]:
            fork(sx, s0)

    def record_projections(streams):
        """The step as independent chains: projection j's materialize, forward,
        dX and dW in order on branch j % len(streams)."""
        s0 = streams[0]

        def fork(src, dst):
            e = torch.cuda.Event()
            e.record(src)
            dst.wait_event(e)

        for sx in streams[1:]:
            fork(s0, sx)
        for j, d in enumerate(projs):
            st = streams[j % len(streams)]
            tl.tern_materialize(d["q"], d["theta"], d["packed"], st)
            tl.tern_linear_fwd(d["X"], d["packed"], d["scale"], d["Y"], st)
            tl.tern_linear_bwd_dx(d["dY"], d["packed"], d["scale"], d["dX"], stream=st)
            tl.tern_linear_bwd_dw(d["X"], d["dY"], d["packed"], d["scale"], d["gq"], d["sgrad"], d["ws"], st)
        for sx in streams[1:]:
            fork(sx, s0)

    eager_ms_per_step = ms_per_step
    # per-step times of the eager region (first event of a step to its last)
    last = 0 if layer else -1
    step_ms = [evs[k][0][0].elapsed_time(evs[k][last][4]) for k in range(a.steps)]
    if a.streams == "auto":
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        tiles = lambda m, n: -(-m // 512) * -(-n // 128)   # the forward / dX kernels' items
        if layer:
            items = (sum(tiles(d["n_out"], w.T) for d in projs), sum(tiles(d["n_in"], w.T) for d in projs))
            mode = "3" if min(items) < cus else "1"
        else:
            small = any(min(tiles(d["n_out"], w.T), tiles(d["n_in"], w.T)) < cus for d in projs)
            mode = "p3" if small else "2"
    else:
        mode = a.streams
        if layer and mode.startswith("p"):
            mode = mode[1:]
    by_projection = mode.startswith("p")
    n_streams = int(mode[1:] if by_projection else mode)
    if a.launch == "graph":
        # one step recorded on a side stream (plus branch streams), replayed as
        # one launch per step
        gs = torch.cuda.Stream()
        gs.wait_stream(stream)
        branches = [torch.cuda.Stream() for _ in range(n_streams - 1)]
        tl.tern_graph_begin(gs)
        try:
            if layer:
                record_layer([gs] + branches)
            else:
                (record_projections if by_projection else record_dag)([gs] + branches)
        finally:
            graph = tl.tern_graph_end(gs)
        try:
            for _ in range(a.warmup):
                tl.tern_graph_launch(graph, gs)
            torch.cuda.synchronize()
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(a.steps)]
            ready_events([g0, g1] + [e for pair in rev for e in pair], gs)
            g0.record(gs)
            for k in range(a.steps):
                rev[k][0].record(gs)
                tl.tern_graph_launch(graph, gs)
                rev[k][1].record(gs)
            g1.record(gs)
            torch.cuda.synchronize()
            ms_per_step = g0.elapsed_time(g1) / a.steps
            step_ms = [e0.elapsed_time(e1) for e0, e1 in rev]
            power = None if a.no_power else board_power(lambda: tl.tern_graph_launch(graph, gs), ms_per_step)
        finally:
            tl.tern_graph_destroy(graph)
    elif not a.no_power:
        power = board_power(step, ms_per_step)
    else:
        power = None

    # per step, summed over projections: the mean over the timed steps, and
    # each part's median over the steps
    per_step = {p: [0.0] * a.steps for p in PARTS}
    for k in range(a.steps):
        for j in range(1 if layer else len(projs)):
            for pi, pname in enumerate(PARTS):
                per_step[pname][k] += evs[k][j][pi].elapsed_time(evs[k][j][pi + 1])
    part_ms = {p: sum(v) / a.steps for p, v in per_step.items()}
    part_med = {p: statistics.median(v) for p, v in per_step.items()}

    flops_step = w.flops
    gemm_flops = {p: 2.0 * w.T * w.sum_in_out for p in ("fwd", "bwd_dx", "bwd_dw")}
    tflops = flops_step / (ms_per_step * 1e-3) / 1e12
    tokens_per_s = w.T / (ms_per_step * 1e-3)
    dt = w.act
    peak = PEAK_TFLOPS[dt]

    # dominant kernel: the GEMM entry point with the largest share of the step
    dom = max(("fwd", "bwd_dx", "bwd_dw"), key=lambda p: part_ms[p])
    dom_kernels = {"fwd": "gemm_rd_kernel<MODE_FWD> (tern_layer_fwd)" if layer else
                   "gemm_rd_kernel<MODE_FWD> (tern_linear_fwd)",
                   "bwd_dx": "gemm_rd_kernel<MODE_DX> (tern_layer_bwd_dx)" if layer else
                   "gemm_rd_kernel<MODE_DX> (tern_linear_bwd_dx)",
                   "bwd_dw": "gemm_dw_kernel + dw_reduce + sgrad_reduce (tern_layer_bwd_dw)" if layer else
                   "gemm_dw_kernel + dw_reduce + sgrad_reduce (tern_linear_bwd_dw)"}[dom]
    achieved = gemm_flops[dom] / (part_ms[dom] * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            ent = tr.get("entries", {}).get(f"{w.name}/{dom}")
            if ent and tr.get("kernel_src_sha256_16") == kernel_src_hash():
                traffic = ent["bytes_per_step"]
        except Exception:  # noqa: BLE001 - a stale or malformed file means no counter data
            traffic = None
    es = 2 if dt == "bf16" else 4
    alg_bytes = {p: sum(algorithmic_bytes(p, w.T, i, o, es) for _, i, o in w.projs) for p in PARTS}
    alg_gbs = alg_bytes[dom] / (part_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": dom_kernels,
                "flops_per_step": gemm_flops[dom], "ms_per_step": round(part_ms[dom], 4),
                "ms_per_step_median": round(part_med[dom], 4),
                "alg_bytes_per_step": alg_bytes[dom], "alg_hbm_gbs": round(alg_gbs, 1),
                "alg_hbm_frac": round(alg_gbs / PEAK_HBM_GBS, 4)}
    if traffic is not None:
        # the same kernel against the HBM roof: its counted bytes over its time
        gbs = traffic / (part_ms[dom] * 1e-3) / 1e9
        roofline.update(hbm_gbs=round(gbs, 1), hbm_peak_gbs=PEAK_HBM_GBS, hbm_frac=round(gbs / PEAK_HBM_GBS, 4))

    if a.copy_calibration:
        # one elementwise kernel per copy: reads and writes COPY_BYTES once
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.mul(src, 1, out=dst)
        torch.cuda.synchronize()
        del src, dst

    vendor = None if a.no_vendor_gemm else vendor_gemm(w, projs, peak)

    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(w, projs, a.cpu_rows, a.cpu_cols, a.cpu_1t_div)

    line = {
        "metric": "ternary-linear fwd+bwd TFLOP/s and tokens/s at d=2048; % of MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T,
                   "projections": [[n, i, o] for n, i, o in w.projs],
                   "theta": w.theta, "q": w.q_law, "scale": w.scale_law, "act": w.act,
                   "launch": (f"hipgraph, {n_streams} branch(es)" + (" by projection" if by_projection else ""))
                   if a.launch == "graph" else "eager",
                   "api": "tern_layer_* (one call per product for all projections)" if layer
                   else "single-projection calls"},
        "eager_ms_per_step": round(eager_ms_per_step, 4),
        "tokens_per_s": round(tokens_per_s, 1),
        "mfma_frac": round(tflops / peak, 4),
        "flops_per_step": flops_step,
        "part_ms_per_step": {k: round(v, 4) for k, v in part_ms.items()},
        "part_ms_median": {k: round(v, 4) for k, v in part_med.items()},
        "step_stats": step_stats(step_ms, flops_step, w.T, peak),
        "part_alg_hbm_gbs": {p: round(alg_bytes[p] / (part_ms[p] * 1e-3) / 1e9, 1) for p in PARTS},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "vendor_gemm": vendor,
        "power": power if power is None else dict(power, tflop_per_j=round(tflops / power["mean_w"], 4),
                                                 j_per_step=round(power["mean_w"] * ms_per_step * 1e-3, 4)),
    }
    print(json.dumps(line), flush=True)


def power_sensor():
    """The board's power sensor (amdgpu hwmon power1_input, microwatts), or None."""
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input")):
        try:
            int(open(f).read())
            return f
        except (OSError, ValueError):
            continue
    return None


def board_power(run_once, step_ms, seconds=1.5):
    """Mean board power while the step repeats for about `seconds`: a host
    thread reads the sensor every 5 ms; the first 30 % of the window, while the
    clock settles, is left out.  Also the cap (power1_cap).  None without a
    readable sensor."""
    import threading

    import torch

    f = power_sensor()
    if f is None:
        return None
    read = lambda: int(open(f).read()) / 1e6  # noqa: E731
    try:
        cap = int(open(f.replace("power1_input", "power1_cap")).read()) / 1e6
    except (OSError, ValueError):
        cap = None
    torch.cuda.synchronize()
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            samples.append((time.time(), read()))
            time.sleep(0.005)

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    batch = max(1, int(50.0 / max(step_ms, 1e-3)))   # about 50 ms of steps per synchronisation
    t0 = time.time()
    n = 0
    while time.time() - t0 < seconds:
        for _ in range(batch):
            run_once()
        n += batch
        torch.cuda.synchronize()
    t1 = time.time()
    stop.set()
    th.join()
    win = [v for t, v in samples if t0 + 0.3 * (t1 - t0) <= t <= t1]
    if not win:
        return None
    return {"mean_w": round(statistics.mean(win), 1), "max_w": round(max(win), 1), "cap_w": cap,
            "window_s": round(t1 - t0, 2), "steps": n, "samples": len(win), "sensor": f}


def vendor_gemm(w, projs, peak, reps=5):
    """Context, not this library: the vendor's dense bf16 GEMM (torch.mm, which
    dispatches to hipBLASLt) on the step's three products for every projection,
    with a dense bf16 weight matrix W[r][c] = bf16(scale[c] * tern[r][c]) and
    fp32 outputs like the library's: Y = X W, dX = dY W^T (W^T stored
    contiguous), G = X^T dY (X^T a transposed view: both operands token-major,
    as the library reads them).  No materialize, no scale epilogue, no gq or
    sgrad.  Timed as one sequence of the three products per repetition, after
    two untimed ones; each product's median over the repetitions."""
    import torch

    mats = []
    for d in projs:
        q = d["q"]
        tern = (q >= d["theta"]).to(torch.float32) - (q <= -d["theta"]).to(torch.float32)
        W = (tern * d["scale"][None, :]).to(torch.bfloat16)
        mats.append((d["X"], d["dY"], W, W.t().contiguous()))
        del tern
    f32 = torch.float32

    def fwd():
        for X, dY, W, WT in mats:
            torch.mm(X, W, out_dtype=f32)

    def dx():
        for X, dY, W, WT in mats:
            torch.mm(dY, WT, out_dtype=f32)

    def dw():
        for X, dY, W, WT in mats:
            torch.mm(X.t(), dY, out_dtype=f32)

    parts = {"fwd": fwd, "bwd_dx": dx, "bwd_dw": dw}
    try:
        for _ in range(2):
            for f in parts.values():
                f()
        torch.cuda.synchronize()
    except RuntimeError as e:  # an mm with out_dtype the build does not offer
        return {"error": str(e).splitlines()[0][:200]}
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
          for k in parts}
    for i in range(reps):
        for k, f in parts.items():
            ev[k][i][0].record()
            f()
            ev[k][i][1].record()
    torch.cuda.synchronize()
    med = {k: statistics.median(a.elapsed_time(b) for a, b in ev[k]) for k in parts}
    ms = sum(med.values())
    tf = 3 * 2.0 * w.T * w.sum_in_out / (ms * 1e-3) / 1e12
    del mats
    torch.cuda.empty_cache()
    return {"kind": "dense bf16 torch.mm (hipBLASLt), fp32 out, same shapes, context only",
            "value": round(tf, 2), "unit": "TFLOP/s", "frac": round(tf / peak, 4),
            "ms_per_step": round(ms, 4), "part_ms_median": {k: round(v, 4) for k, v in med.items()},
            "reps": reps}


def algorithmic_bytes(part: str, T: int, n_in: int, n_out: int, es: int) -> float:
    """HBM bytes one entry point must move for one projection: its inputs read
    once, its outputs written once (activations es bytes, tern 1/4 byte per
    weight, scale, Y / dX / gq / sgrad fp32; q one byte per weight)."""
    w = n_in * n_out
    if part == "materialize":
        return 1.0 * w + 0.25 * w
    if part == "fwd":
        return es * T * n_in + 0.25 * w + 4 * n_out + 4 * T * n_out
    if part == "bwd_dx":
        return es * T * n_out + 0.25 * w + 4 * n_out + 4 * T * n_in
    return es * T * (n_in + n_out) + 0.25 * w + 4 * n_out + 4 * w + 4 * n_out   # bwd_dw


def step_stats(step_ms, flops, T, peak):
    """Median, min, max and spread of the per-step times, with the rates at the
    median."""
    s = sorted(step_ms)
    med = statistics.median(s)
    q = lambda f: s[min(len(s) - 1, max(0, int(round(f * (len(s) - 1)))))]
    return {"n": len(s), "median_ms": round(med, 4), "min_ms": round(s[0], 4), "max_ms": round(s[-1], 4),
            "p10_ms": round(q(0.1), 4), "p90_ms": round(q(0.9), 4),
            "spread_pct": round(100.0 * (q(0.9) - q(0.1)) / med, 2),
            "tflops_at_median": round(flops / (med * 1e-3) / 1e12, 3),
            "mfma_frac_at_median": round(flops / (med * 1e-3) / 1e12 / peak, 4),
            "tokens_per_s_at_median": round(T / (med * 1e-3), 1)}


def cpu_baseline(w, projs, n_rows, n_cols, div_1t=16):
    """The oracle, as it stands, on a bounded sample of the same workload:
    n_rows token rows of Y and dX and n_cols output columns of gq / sgrad per
    projection.  Reported as the oracle's throughput (TFLOP/s) and the tokens/s
    of a full step at that rate."""
    import oracle
    import synth

    o = oracle.get()
    flops = 0.0
    t0 = time.perf_counter()
    for i, d in enumerate(projs):
        p = d["host"]
        rows = synth.sample_indices(synth.stream_seed(91, w.config_id, i, 0), n_rows, w.T)
        cols = synth.sample_indices(synth.stream_seed(91, w.config_id, i, 1), n_cols, d["n_out"])
        o.linear_fwd(p.X, p.q, p.theta, p.scale, rows=rows)
        o.linear_dx(p.dY, p.q, p.theta, p.scale, rows=rows)
        o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, cols=cols)
        flops += 2.0 * 2 * rows.size * d["n_in"] * d["n_out"] + 2.0 * w.T * d["n_in"] * cols.size
    sec = time.perf_counter() - t0
    rate = flops / sec
    full_s = w.flops / rate
    cores = o.num_threads()
    # the same oracle on one thread, on 1/div_1t of the sample
    r1, c1 = max(1, n_rows // div_1t), max(1, n_cols // div_1t)
    o.set_num_threads(1)
    try:
        flops1 = 0.0
        t1 = time.perf_counter()
        for i, d in enumerate(projs):
            p = d["host"]
            rows = synth.sample_indices(synth.stream_seed(92, w.config_id, i, 0), r1, w.T)
            cols = synth.sample_indices(synth.stream_seed(92, w.config_id, i, 1), c1, d["n_out"])
            o.linear_fwd(p.X, p.q, p.theta, p.scale, rows=rows)
            o.linear_dx(p.dY, p.q, p.theta, p.scale, rows=rows)
            o.linear_wgrad(p.X, p.dY, p.q, p.theta, p.scale, cols=cols)
            flops1 += 2.0 * 2 * rows.size * d["n_in"] * d["n_out"] + 2.0 * w.T * d["n_in"] * cols.size
        sec1 = time.perf_counter() - t1
    finally:
        o.set_num_threads(cores)
    rate1 = flops1 / sec1
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_rows} token rows of Y and dX and {n_cols} output columns of gq/sgrad per "
                      f"projection, all {len(projs)} projections of {w.name}; {sec:.1f}s",
            "seconds": round(sec, 2), "extrapolated_step_s": round(full_s, 1),
            "tokens_per_s": round(w.T / full_s, 3),
            "value_1thread": round(rate1 / 1e12, 6),
            "sample_1thread": f"{r1} token rows and {c1} columns per projection; {sec1:.1f}s",
            "extrapolated_step_s_1thread": round(w.flops / rate1, 1),
            "thread_speedup": round(rate / rate1, 2)}


if __name__ == "__main__":
    main()
