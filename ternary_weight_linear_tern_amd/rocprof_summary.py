"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m ternary_weight_linear_tern_amd.rocprof_summary stats  <kernel_stats.csv> [title]
    python -m ternary_weight_linear_tern_amd.rocprof_summary timed  <kernel_trace.csv> <last> [title]
    python -m ternary_weight_linear_tern_amd.rocprof_summary counters <counter_collection.csv> [title]
    python -m ternary_weight_linear_tern_amd.rocprof_summary ratios <counter_collection.csv> [title]
    python -m ternary_weight_linear_tern_amd.rocprof_summary l2 <counter_collection.csv> [title]
    python -m ternary_weight_linear_tern_amd.rocprof_summary traffic <reqsize_counter_collection.csv> \\
        <write_counter_collection.csv> <workload> <dispatch_steps> [sources ...]

`traffic` attributes the read bytes (from TCC_EA0_RDREQ_{32B,64B,128B}) and
WRITE_SIZE to the library's entry points, checks both against the calibration
copy (bench.py --copy-calibration: 1 GiB read + 1 GiB written by one
elementwise multiply-by-one kernel per copy) and scales by it, divides by the
number of profiled steps, and writes
profiles/traffic_counters.json, which bench.py reports as roofline.traffic
while the code of the kernels and of the planner (which sets their launch
shapes) is unchanged.
"""
from __future__ import annotations

import csv
import re
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KIB = (1 << 30) / 1024.0


def kernel_code_hash(*paths: str) -> str:
    """First 16 hex digits of the SHA-256 of C++/HIP sources (in the order
    given) with their comments and blank lines removed and each line's
    surrounding whitespace stripped, so that the hash names the code whose
    counters were taken, not its comments.  Without paths: the kernels and
    the planner and the layer calls that set their launch shapes (tile,
    split-K, reduce rows, item walk)."""
    if not paths:
        paths = tuple(os.path.join(PKG, "csrc", f)
                      for f in ("tern_kernels.hip", "tern_plan.h", "tern_plan.cpp", "tern_layer.cpp"))
    h = hashlib.sha256()
    for path in paths:
        text = open(path, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*", "", l).strip() for l in text.splitlines())
        h.update("\n".join(l for l in lines if l).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def entry_of(kernel: str) -> str | None:
    k = kernel
    if "materialize_kernel" in k or "materialize_group_kernel" in k or "derive_kernel" in k:
        return "materialize"
    if "gemm_dw_kernel" in k:
        return "bwd_dw"
    if "gemm" in k:
        # gemm_rd_kernel<MODE, ACC> and gemm_kernel<BF, MODE, BM>: the mode is
        # the first template argument of the former, the second of the latter
        m = re.search(r"gemm_rd_kernel<(\d)", k) or re.search(r"gemm_kernel<\w+, (\d)", k)
        mode = m.group(1) if m else None
        return {"0": "fwd", "1": "bwd_dx", "2": "bwd_dw"}.get(mode)
    if "dw_reduce" in k or "sgrad_reduce" in k:
        return "bwd_dw"
    return None


def stats(path: str, title: str = "") -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# {title}" if title else "# kernel stats", "",
           "| kernel | calls | total ms | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['TotalDurationNs'])/1e6:.3f} | "
                   f"{float(r['AverageNs'])/1e3:.1f} | {float(r['MinNs'])/1e3:.1f} | {float(r['MaxNs'])/1e3:.1f} | "
                   f"{float(r['Percentage']):.2f} |")
    return "\n".join(out)


def _counter_sums(path: str, counter: str):
    per_kernel = defaultdict(float)
    per_kernel_n = defaultdict(int)
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        name = r["Kernel_Name"]
        per_kernel[name] += float(r["Counter_Value"])
        per_kernel_n[name] += 1
    return per_kernel, per_kernel_n


def read_kib_by_size(csv_path: str):
    """Per kernel, the memory read bytes (KiB, summed over dispatches) from
    the L2's read requests by size: 32 TCC_EA0_RDREQ_32B + 64 TCC_EA0_RDREQ_64B
    + 128 TCC_EA0_RDREQ_128B.  (FETCH_SIZE weights every request that is not
    32 bytes as 64 bytes, so it reads 128-byte requests at half their size.)"""
    n32, cnt = _counter_sums(csv_path, "TCC_EA0_RDREQ_32B_sum")
    n64, _ = _counter_sums(csv_path, "TCC_EA0_RDREQ_64B_sum")
    n128, _ = _counter_sums(csv_path, "TCC_EA0_RDREQ_128B_sum")
    out = {}
    for k in set(n32) | set(n64) | set(n128):
        out[k] = (32 * n32.get(k, 0.0) + 64 * n64.get(k, 0.0) + 128 * n128.get(k, 0.0)) / 1024.0
    return out, cnt


def traffic(read_csv: str, write_csv: str, workload: str, steps: int, kernel_src: str | None = None):
    """HBM bytes per step of each entry point: reads from the request sizes
    (read_kib_by_size), writes from WRITE_SIZE, each checked against the 1 GiB
    calibration copies (and scaled by what they read, should it not be 1)."""
    f, fn = read_kib_by_size(read_csv)
    w, wn = _counter_sums(write_csv, "WRITE_SIZE")
    copy_f = [v / fn[k] for k, v in f.items() if "MulFunctor" in k]
    copy_w = [v / wn[k] for k, v in w.items() if "MulFunctor" in k]
    # the calibration copies are the only multiply kernels in the run
    fscale = COPY_KIB / max(copy_f) if copy_f else 1.0
    wscale = COPY_KIB / max(copy_w) if copy_w else 1.0
    ent = defaultdict(lambda: {"fetch_kib": 0.0, "write_kib": 0.0})
    lines = [f"# HBM traffic per step, {workload} ({steps} profiled steps)", "",
             f"calibration: a 1 GiB copy reads {1 / fscale:.4f} GiB by request sizes and writes "
             f"{1 / wscale:.4f} GiB by WRITE_SIZE; scale factors {fscale:.4f} / {wscale:.4f}", "",
             "| kernel | dispatches | read KiB/dispatch | WRITE KiB/dispatch |", "|---|---|---|---|"]
    for k in sorted(set(f) | set(w)):
        lines.append(f"| {k[:80]} | {fn.get(k, 0)} | {f.get(k, 0)/max(fn.get(k, 1),1):.0f} | "
                     f"{w.get(k, 0)/max(wn.get(k, 1),1):.0f} |")
        e = entry_of(k)
        if e:
            ent[e]["fetch_kib"] += f.get(k, 0.0)
            ent[e]["write_kib"] += w.get(k, 0.0)
    out = {"kernel_src_sha256_16": None, "entries": {}, "calibration": {"fetch": fscale, "write": wscale}}
    if kernel_src:
        out["kernel_src_sha256_16"] = kernel_code_hash(*kernel_src) if isinstance(kernel_src, (list, tuple)) \
            else kernel_code_hash(kernel_src)
    lines += ["", "| entry point | HBM read MB/step | HBM write MB/step |", "|---|---|---|"]
    for e, v in sorted(ent.items()):
        rd = v["fetch_kib"] * fscale * 1024 / steps
        wr = v["write_kib"] * wscale * 1024 / steps
        out["entries"][f"{workload}/{e}"] = {"read_bytes_per_step": rd, "write_bytes_per_step": wr,
                                             "bytes_per_step": rd + wr}
        lines.append(f"| {e} | {rd/1e6:.1f} | {wr/1e6:.1f} |")
    return out, "\n".join(lines)


def timed(trace_csv: str, last: int, title: str = "") -> str:
    """Per kernel, the mean duration of its last `last` dispatches in a
    --kernel-trace CSV: the dispatches of the region bench.py keeps (its
    eager region runs twice and reports the second), which are the ones its
    events time, without the warm-up and first-region dispatches that the
    --stats average includes."""
    per = defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        per[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out = [f"# {title}" if title else "# last dispatches", "",
           f"| kernel | dispatches | mean of the last {last}, us |", "|---|---|---|"]
    for name, ds in sorted(per.items(), key=lambda kv: -sum(e - s for s, e in kv[1])):
        ds.sort()
        tail = ds[-last:]
        mean = sum(e - s for s, e in tail) / len(tail) / 1e3
        out.append(f"| {name[:80]} | {len(ds)} | {mean:.1f} |")
    return "\n".join(out)


def l2(path: str, title: str = "") -> str:
    """Per kernel, over its dispatches: the L2 hit rate (TCC_HIT / (TCC_HIT +
    TCC_MISS)) and the mean L1-to-L2 read latency in cycles
    (TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ)."""
    tot = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(path)):
        tot[r["Kernel_Name"]][r["Counter_Name"]] += float(r["Counter_Value"])
    out = [f"# {title}" if title else "# L2", "", "| kernel | L2 hit % | L1->L2 read latency (cycles) | L1->L2 reads |",
           "|---|---|---|---|"]
    for name, c in sorted(tot.items()):
        h, m = c.get("TCC_HIT_sum", 0.0), c.get("TCC_MISS_sum", 0.0)
        lat, req = c.get("TCP_TCC_READ_REQ_LATENCY_sum", 0.0), c.get("TCP_TCC_READ_REQ_sum", 0.0)
        hit = f"{100 * h / (h + m):.1f}" if h + m else "-"
        l = f"{lat / req:.0f}" if req else "-"
        out.append(f"| {name[:70]} | {hit} | {l} | {req:.3g} |")
    return "\n".join(out)


XCDS = 8          # GRBM_GUI_ACTIVE is reported summed over the 8 XCD instances
SIMDS = 256 * 4   # MI355X: 256 compute units x 4 SIMDs


def counters(path: str, title: str = "") -> str:
    """Per kernel, medians over its dispatches: duration, shader clock
    (GRBM_GUI_ACTIVE per XCD over the dispatch's time), MFMA busy
    (SQ_VALU_MFMA_BUSY_CYCLES over SIMD cycles, rocprofv3's MfmaUtil), bf16
    matrix TFLOP/s from SQ_INSTS_VALU_MFMA_MOPS_BF16 (512 flops per op) and the
    share of wave cycles waiting on LDS.  The counter window of a dispatch
    outlasts kernels of a few tens of microseconds, so their clock (and MFMA
    busy) figures are not meaningful; they are marked."""
    import statistics
    per = defaultdict(lambda: defaultdict(float))
    secs = {}
    for r in csv.DictReader(open(path)):
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        secs[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    rows = defaultdict(list)
    for key, c in per.items():
        sec = secs[key]
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        rows[key[1]].append(dict(
            sec=sec, clk=gui / sec / 1e9 if sec else 0.0,
            busy=100.0 * c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * SIMDS) if gui else 0.0,
            tf=c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512.0 / sec / 1e12 if sec else 0.0,
            wl=100.0 * c.get("SQ_WAIT_INST_LDS", 0.0) / c["SQ_WAVE_CYCLES"] if c.get("SQ_WAVE_CYCLES") else 0.0))
    out = [f"# {title}" if title else "# kernel counters", "",
           "| kernel | dispatches | median us | clock GHz | MFMA busy % | bf16 MFMA TFLOP/s | LDS wait % of wave cycles |",
           "|---|---|---|---|---|---|---|"]
    for name, rs in sorted(rows.items(), key=lambda kv: -sum(r["sec"] for r in kv[1])):
        med = {k: statistics.median(r[k] for r in rs) for k in rs[0]}
        short = med["sec"] < 50e-6
        clk = "(short)" if short else f"{med['clk']:.2f}"
        busy = "(short)" if short else f"{med['busy']:.1f}"
        out.append(f"| {name[:80]} | {len(rs)} | {1e6 * med['sec']:.1f} | {clk} | {busy} | {med['tf']:.0f} | "
                   f"{med['wl']:.1f} |")
    return "\n".join(out)


def ratios(path: str, title: str = "") -> str:
    """Per kernel, the median over its dispatches of every counter in the
    file divided by SQ_WAVE_CYCLES (wave-cycle shares), and of the icache
    miss rate when SQC_ICACHE_HITS / SQC_ICACHE_MISSES are present."""
    import statistics
    per = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(path)):
        per[(r["Dispatch_Id"], r["Kernel_Name"])][r["Counter_Name"]] += float(r["Counter_Value"])
    rows = defaultdict(list)
    for (_, name), c in per.items():
        d = {}
        w = c.get("SQ_WAVE_CYCLES")
        for k, v in c.items():
            if w and k.startswith("SQ_") and k != "SQ_WAVE_CYCLES":
                d[k + " / SQ_WAVE_CYCLES"] = v / w
        if "SQC_ICACHE_HITS" in c:
            tot = c["SQC_ICACHE_HITS"] + c.get("SQC_ICACHE_MISSES", 0.0)
            d["icache miss rate"] = c.get("SQC_ICACHE_MISSES", 0.0) / tot if tot else 0.0
        rows[name].append(d)
    keys = sorted({k for rs in rows.values() for d in rs for k in d})
    out = [f"# {title}" if title else "# counter ratios", "", "| kernel | " + " | ".join(keys) + " |",
           "|---|" + "---|" * len(keys)]
    for name, rs in sorted(rows.items()):
        if not any(rs):
            continue
        vals = [f"{statistics.median(d.get(k, 0.0) for d in rs):.4f}" for k in keys]
        out.append(f"| {name[:60]} | " + " | ".join(vals) + " |")
    return "\n".join(out)


if __name__ == "__main__":
    cmd = sys.argv[1]
    if cmd == "stats":
        print(stats(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
    elif cmd == "timed":
        print(timed(sys.argv[2], int(sys.argv[3]), sys.argv[4] if len(sys.argv) > 4 else ""))
    elif cmd == "ratios":
        print(ratios(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
    elif cmd == "l2":
        print(l2(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
    elif cmd == "counters":
        print(counters(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else ""))
    elif cmd == "traffic":
        src = sys.argv[6:] if len(sys.argv) > 6 else \
            [os.path.join(PKG, "csrc", f) for f in ("tern_kernels.hip", "tern_plan.h", "tern_plan.cpp", "tern_layer.cpp")]
        data, text = traffic(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]), src)
        print(text)
        dst = os.path.join(ROOT, "profiles", "traffic_counters.json")
        os.makedirs(os.path.dirname(dst), exist_ok=True)
        old = json.load(open(dst)) if os.path.exists(dst) else {}
        if old.get("kernel_src_sha256_16") == data["kernel_src_sha256_16"]:
            old.setdefault("entries", {}).update(data["entries"])
            data["entries"] = old["entries"]
        json.dump(data, open(dst, "w"), indent=1)
    else:
        raise SystemExit(__doc__)
