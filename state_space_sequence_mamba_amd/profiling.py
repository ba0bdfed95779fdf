"""Summaries of rocprofv3 runs of the benchmark (measurement tooling, not part of the scan).

  python -m state_space_sequence_mamba_amd.profiling traffic \\
      --fetch DIR --write DIR --copy-mb 1024 --workload NAME --command "..." --out profiles/X.json

reads the counter CSVs of a FETCH_SIZE run and of a WRITE_SIZE run of `bench.py
--copy-probe-mb N`, calibrates each counter on the plain device copy of N MiB that the
benchmark ran in the same process (known bytes read and written), and writes, per SSD
kernel, the HBM bytes per launch.  The JSON carries a digest of the HIP sources, so the
benchmark reports the figure only while the kernels are unchanged.

  python -m state_space_sequence_mamba_amd.profiling stats --trace DIR

prints per-kernel average durations of a --kernel-trace --stats run.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SSD_KERNELS = ["chunk_state", "chunk_state_seq", "chunk_state_seg", "state_passing", "chunk_scan", "ssd_step", "conv1d_silu",
               "conv1d_silu_step", "bwd_dxdb", "bwd_dc", "bwd_finalize"]
# source file of each kernel; every kernel also depends on the shared headers and the API layer
# (which picks launch shapes)
KERNEL_SOURCE = {"chunk_state": "chunk_state.hip", "chunk_state_seq": "chunk_state.hip",
                 "chunk_state_seg": "chunk_state_seg.hip",
                 "state_passing": "state_passing.hip",
                 "chunk_scan": ["chunk_scan.hip", "chunk_scan_group.hip"], "ssd_step": "ssd_step.hip",
                 "conv1d_silu": "conv1d.hip", "conv1d_silu_step": "conv1d.hip", "bwd_dxdb": "ssd_bwd.hip",
                 "bwd_dc": "ssd_bwd.hip", "bwd_finalize": "ssd_bwd.hip"}
SHARED_SOURCES = ["ssd_common.h", "ssd_launch.h", "cb_tiles.h", "ssd_api.hip"]


def source_digest(kernel):
    """sha256 over the sources one kernel is built and launched from."""
    h = hashlib.sha256()
    src = KERNEL_SOURCE[kernel]
    for name in (src if isinstance(src, list) else [src]) + SHARED_SOURCES:
        h.update(name.encode())
        with open(os.path.join(PKG, "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def kernel_key(name):
    """Map a dispatch's kernel name to a kernel key, 'copy' for copy kernels, else None."""
    if "chunk_scan" in name:
        return "chunk_scan"
    for k in ("chunk_state_seq", "chunk_state_seg", "chunk_state", "state_passing", "ssd_step", "conv1d_silu_step", "conv1d_silu",
              "bwd_dxdb", "bwd_dc", "bwd_finalize"):
        if k + "_kernel" in name:
            return k
    if "copyBuffer" in name or "copy_kernel" in name:
        return "copy"
    return None


def _rows(d):
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    if not out:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    return out


def counter_per_dispatch(d, counter):
    """{kernel key: [value per dispatch]} for one counter (values summed over its instances)."""
    per = {}
    for r in _rows(d):
        if r["Counter_Name"] != counter:
            continue
        key = kernel_key(r["Kernel_Name"])
        if key is None:
            continue
        disp = (r["Dispatch_Id"], key)
        per.setdefault(disp, 0.0)
        per[disp] += float(r["Counter_Value"])
    res = {}
    for (disp, key), v in per.items():
        res.setdefault(key, []).append(v)
    return res


def traffic(args):
    copy_bytes = args.copy_mb * 1024 * 1024
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(args.write, "WRITE_SIZE")
    # the probe copy is the largest "copy" dispatch (other copies are tiny staging copies)
    f_copy = max(fetch.get("copy", [0.0]))
    w_copy = max(write.get("copy", [0.0]))
    if f_copy <= 0 or w_copy <= 0:
        sys.exit("probe copy not found in the counter runs")
    f_scale = copy_bytes / f_copy          # bytes per counter unit (counters report KiB)
    w_scale = copy_bytes / w_copy
    kernels = {}
    for k in SSD_KERNELS:
        if k in fetch and k in write:
            fb = sum(fetch[k]) / len(fetch[k]) * f_scale
            wb = sum(write[k]) / len(write[k]) * w_scale
            kernels[k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes": fb + wb,
                          "dispatches": len(fetch[k]), "source_digest": source_digest(k)}
    out = {"workload": args.workload,
           "copy_probe_bytes": copy_bytes,
           "copy_probe_counter_kib": {"FETCH_SIZE": f_copy, "WRITE_SIZE": w_copy},
           "scale_bytes_per_unit": {"FETCH_SIZE": f_scale, "WRITE_SIZE": w_scale},
           "kernels": kernels, "command": args.command}
    with open(args.out, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def stats(args):
    files = glob.glob(os.path.join(args.trace, "**", "*kernel_stats.csv"), recursive=True)
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Name"].split("(")[0].replace("void ", "")
                print(f"{name:70s} calls {r['Calls']:>5s}  avg {float(r['AverageNs']) / 1000:9.2f} us  "
                      f"{float(r['Percentage']):6.2f} %")


def _bench_line(log):
    """The JSON line bench.py printed in a profiled run's log, or None."""
    if not log or not os.path.exists(log):
        return None
    with open(log) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("{") and '"metric"' in line:
                return json.loads(line)
    return None


def summary(args):
    """Markdown summary of one kernel-trace run: per-kernel calls and average duration, next to
    the per-kernel durations bench.py measured with HIP events in the same process."""
    files = glob.glob(os.path.join(args.trace, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        sys.exit(f"no kernel_stats.csv under {args.trace}")
    rows = []
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            name = r["Name"].split("(")[0].replace("void ", "")
            rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1000.0, float(r["Percentage"])))
    bench = _bench_line(args.log)
    events = {}
    if bench:
        for k, v in bench.get("kernels", {}).items():
            # (bench.py names state_passing over segments after its role; the trace, after its kernel)
            events["state_passing" if k == "state_passing_seg" else k] = v["us"]
        rl = bench.get("roofline", {})
        if rl.get("kernel"):
            # (the decode line carries its kernel's dispatch-event average in the roofline)
            events.setdefault(rl["kernel"], rl.get("kernel_us"))
    out = [f"# Kernel trace: {args.workload} (MI355X, gfx950)", "",
           "Command (from the repository root, TMPDIR=/tmp):", "", f"    {args.command}", "",
           "Summarised with `python -m state_space_sequence_mamba_amd.profiling summary` from the run's "
           "kernel_stats.csv.  The last column is the per-kernel duration bench.py measured with "
           "dispatch-recorded HIP events in a separate, unprofiled run of the same bench.py command "
           "on the same box (the profiler's dispatch interception distorts those events).", "",
           "| kernel | calls | rocprofv3 average (us) | share of GPU time | bench.py HIP-event average (us) |",
           "|---|---|---|---|---|"]
    for name, calls, avg, pct in rows:
        key = kernel_key(name)
        ev = events.get(key) if key else None
        out.append(f"| `{name}` | {calls} | {avg:.2f} | {pct:.1f} % | {'' if ev is None else f'{ev:.2f}'} |")
    if bench:
        out += ["", f"Unprofiled bench.py line: `{bench['ms_per_step']}` ms per step, value {bench['value']:.4g} "
                f"{bench['unit']}, roofline {json.dumps(bench.get('roofline'))}."]
    text = "\n".join(out) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    print(text)


MFMA_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_F32", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES",
                 "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "GRBM_GUI_ACTIVE"]
MFMA_PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}


def mfma(args):
    """Markdown summary of one counter run over MFMA_COUNTERS: per kernel, the matrix-core work
    the hardware counted (the MOPS counters count MFMA operations in units of 512 flops), its
    ratio to the kernel's algorithmic flops, and that work's rate over the kernel's duration
    (dispatch events of the same bench.py run) against the published dense peak."""
    per = {c: counter_per_dispatch(args.pmc, c) for c in MFMA_COUNTERS}
    bench = _bench_line(args.log)
    if not bench:
        sys.exit(f"no bench.py line in {args.log}")
    dtype = bench["dtype"]
    kernels = bench.get("kernels", {})
    # kernel durations from the kernel-trace summary of the same workload (rocprofv3 averages):
    # dispatch events inside a counter run are stretched by the collection
    dur = {}
    with open(args.trace_md) as fh:
        for line in fh:
            cells = [c.strip() for c in line.split("|")]
            if len(cells) > 4 and cells[1].startswith("`"):
                key = kernel_key(cells[1].strip("`"))
                if key and key not in dur:
                    dur[key] = float(cells[3])
    out = [f"# MFMA counters: {args.workload} (MI355X, gfx950)", "",
           "Command (from the repository root, TMPDIR=/tmp):", "", f"    {args.command}", "",
           "Summarised with `python -m state_space_sequence_mamba_amd.profiling mfma` from the run's "
           "counter_collection.csv (counter values summed over their instances, averaged over the "
           "dispatches of each kernel).  Counted MFMA flops = 512 x (SQ_INSTS_VALU_MFMA_MOPS_F32 + "
           "SQ_INSTS_VALU_MFMA_MOPS_BF16) per dispatch; the ratio column divides it by the kernel's "
           "algorithmic flops (causal half of the in-chunk products, C B^T once per group), so values "
           "above 1 are work the kernel spends beyond the algorithm (masked upper halves of diagonal "
           "tiles, C B^T per head).  The rate column divides the counted flops by the kernel's average "
           f"duration in the kernel trace `{os.path.basename(args.trace_md)}` (same workload, unprofiled "
           "by counters; dispatch events inside a counter run are stretched by the collection); the "
           f"peak is the published dense {dtype} MFMA peak "
           f"({MFMA_PEAK_TFLOPS[dtype]} TFLOP/s).  Wait share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wave "
           "cycles spent waiting on an s_waitcnt).", "",
           "| kernel | dispatches | counted MFMA GFLOP | algorithmic GFLOP | ratio | trace duration (us) | "
           "counted MFMA TFLOP/s | of peak | wait share | SQ_VALU_MFMA_BUSY_CYCLES | SQ_BUSY_CYCLES | "
           "GRBM_GUI_ACTIVE |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    avg = lambda c, k: (sum(per[c][k]) / len(per[c][k])) if k in per[c] else 0.0  # noqa: E731
    for k in SSD_KERNELS:
        if k not in per["SQ_WAVE_CYCLES"] or k not in kernels:
            continue
        mops = avg("SQ_INSTS_VALU_MFMA_MOPS_F32", k) + avg("SQ_INSTS_VALU_MFMA_MOPS_BF16", k)
        flops = 512.0 * mops
        alg = kernels[k].get("alg_flops", 0)
        us = dur.get(k, 0.0)
        rate = flops / (us * 1e-6) / 1e12 if us else 0.0
        wait = avg("SQ_WAIT_INST_ANY", k) / max(avg("SQ_WAVE_CYCLES", k), 1.0)
        out.append(f"| {k} | {len(per['SQ_WAVE_CYCLES'][k])} | {flops / 1e9:.3f} | {alg / 1e9:.3f} | "
                   f"{(flops / alg) if alg else float('nan'):.2f} | {us:.2f} | {rate:.1f} | "
                   f"{rate / MFMA_PEAK_TFLOPS[dtype] * 100:.1f} % | {wait * 100:.0f} % | "
                   f"{avg('SQ_VALU_MFMA_BUSY_CYCLES', k):.4g} | {avg('SQ_BUSY_CYCLES', k):.4g} | "
                   f"{avg('GRBM_GUI_ACTIVE', k):.4g} |")
    text = "\n".join(out) + "\n"
    with open(args.out, "w") as fh:
        fh.write(text)
    print(text)


def workload_slug(name):
    return "_".join(name.lower().split())


def load_traffic(workload_slug, kernel):
    """HBM bytes per launch of `kernel` from the committed summary, or None (missing/stale)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_slug}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    k = t.get("kernels", {}).get(kernel)
    if k is None or k.get("source_digest") != source_digest(kernel):
        return None
    return k["bytes"]


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mb", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", default="")
    t.add_argument("--out", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--trace", required=True)
    m = sub.add_parser("summary")
    m.add_argument("--trace", required=True)
    m.add_argument("--log", default="")
    m.add_argument("--workload", required=True)
    m.add_argument("--command", required=True)
    m.add_argument("--out", required=True)
    f = sub.add_parser("mfma")
    f.add_argument("--pmc", required=True)
    f.add_argument("--log", required=True)
    f.add_argument("--trace-md", required=True)
    f.add_argument("--workload", required=True)
    f.add_argument("--command", required=True)
    f.add_argument("--out", required=True)
    a = ap.parse_args()
    {"traffic": traffic, "stats": stats, "summary": summary, "mfma": mfma}[a.cmd](a)


if __name__ == "__main__":
    main()
