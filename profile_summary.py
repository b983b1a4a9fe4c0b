"""Summaries of rocprofv3 runs of bench.py, written under profiles/.

    python profile_summary.py trace   <trace dir> <out.md> --command "<command that made it>"
    python profile_summary.py traffic <FETCH_SIZE dir> <WRITE_SIZE dir> <copy FETCH_SIZE dir>
                                      <copy WRITE_SIZE dir> <out.json> <out.md> --command "..." [...]
    python profile_summary.py sq      <counter dir> [<counter dir> ...] <out.md> --kernel <name prefix>
                                      --grid <work-items> --command "..." [...]

`trace` groups the dispatches of a `--kernel-trace` CSV by kernel, grid and
workgroup size (duration = end - start timestamp).  `traffic` turns the
FETCH_SIZE and WRITE_SIZE readings (KiB per dispatch) into HBM bytes per launch,
each scaled by what the same counter reads for `bench.py --only copy` (five
copies of exactly 256 MiB each way), and records them per named launch in a
JSON file that bench.py reads for `roofline.traffic` while the kernel's source
digest still matches.  `sq` averages the SQ counters of one kernel launch shape
over the second half of its dispatches (after bench.py's settle phases).
"""
import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "block_scaled_precision_requant_amd", "csrc")
COPY_BYTES = 256 * 2 ** 20

# Source files each kernel family is built from (the digest bench.py checks).
SOURCES = {
    "gemm_kernel": ["gemm.hip", "bsr_internal.h", "bsr_geometry.h"],
    "split_reduce_kernel": ["gemm.hip", "bsr_internal.h", "bsr_geometry.h"],
    "requant_w_kernel": ["requant.hip", "bsr_internal.h", "bsr_geometry.h"],
    "requant_a_kernel": ["requant.hip", "bsr_internal.h", "bsr_geometry.h"],
    "silu_requant": ["requant.hip", "bsr_internal.h", "bsr_geometry.h"],
    "quant_": ["requant.hip", "bsr_internal.h", "bsr_geometry.h"],
    "gemv_": ["gemv.hip", "bsr_internal.h", "bsr_geometry.h"],
    "w4a16_": ["w4a16.hip", "bsr_internal.h", "bsr_geometry.h"],
}


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name):
    """Kernel name without the namespace and argument list."""
    base = name.replace("(anonymous namespace)::", "").split("(")[0]
    for prefix in ("void ", "bsr::gemm_kernels::", "bsr::"):
        base = base.replace(prefix, "")
    return base.strip()


def family(name):
    s = short_name(name)
    for key in SOURCES:
        if s.startswith(key):
            return key
    return None


def _rows(directory, suffix):
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not files:
        sys.exit(f"no *{suffix} under {directory}")
    for f in files:
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def _field(row, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(names)


def _grid(row):
    """Grid in work-items and workgroup size of a CSV row."""
    g = int(float(_field(row, "Grid_Size_X", "Grid_Size")))
    w = int(float(_field(row, "Workgroup_Size_X", "Workgroup_Size")))
    return g, w


def cmd_trace(args):
    groups = defaultdict(list)
    for row in _rows(args.dir, "kernel_trace.csv"):
        name = short_name(row["Kernel_Name"])
        g, w = _grid(row)
        groups[(name, g, w)].append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    lines = ["# Kernel trace: " + args.title, "", "Command (from /tmp, one MI355X):", "", "```", args.command, "```", "",
             "Durations per dispatch (end - start timestamp), grouped by kernel and launch shape; every dispatch of",
             "the run is counted (settle phases, warm-up, timed steps, bursts).", "",
             "| kernel | grid (WGs x threads) | calls | avg us | min us | max us | total ms |",
             "|---|---|---|---|---|---|---|"]
    for (name, g, w), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{name}` | {g // w} x {w} | {len(d)} | {sum(d) / len(d):.2f} | {min(d):.2f} | "
                     f"{max(d):.2f} | {sum(d) / 1e3:.2f} |")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(args.out)


def _counter(directory, counter):
    """{(name, grid, wg): [per-dispatch values]} of one counter."""
    per = defaultdict(lambda: defaultdict(float))
    for row in _rows(directory, "counter_collection.csv"):
        if row["Counter_Name"] != counter:
            continue
        g, w = _grid(row)
        key = (row["Kernel_Name"], g, w)
        per[key][row.get("Dispatch_Id") or row.get("Correlation_Id")] += float(row["Counter_Value"])
    return {k: list(v.values()) for k, v in per.items()}


def _copy_scale(directory, counter):
    vals = [x for (name, g, w), v in _counter(directory, counter).items() if "copyBuffer" in name for x in v]
    if not vals:
        sys.exit(f"no copy dispatches with {counter} under {directory}")
    kib = sorted(vals)[len(vals) // 2]   # median: every copy moves the same bytes
    return kib, COPY_BYTES / (kib * 1024.0)


def default_named():
    """The launches bench.py's counters are summarized for, by workload: the
    prefill GEMM (256 x 128 tiles of 512 lanes: every prefill workload's M is a
    multiple of 256), the weight requant (one
    32-element block per lane, 256 lanes per workgroup) and the activation
    requant (four lanes per block, two 8-element chunks per lane), with their
    algorithmic bytes per launch."""
    sys.path.insert(0, ROOT)
    from block_scaled_precision_requant_amd import inputs
    named = {}
    for wl in ("large", "dense_ffn", "attn_proj"):
        for p in inputs.workload(wl).projections:
            m, n, k = p.m, p.n, p.k
            tag = p.name
            gemm_grid = math.ceil(m / 256) * math.ceil(n / 128) * 512
            named[f"gemm_kernel|{tag}"] = dict(
                kernel="gemm_kernel<256, 128, 64, 64, 1, 1, 2, false>", grid=gemm_grid,
                workload=f"GEMM {m}x{n}x{k} ({tag})",
                alg=m * k + n * k + (m + n) * (k // 32) * 4 + 2 * m * n)
            named[f"requant_w_kernel|{tag}"] = dict(
                kernel="requant_w_kernel", grid=math.ceil(n * k // 32 / 256) * 256,
                workload=f"weight requant {n}x{k} ({tag})", alg=n * k * 27 // 16)
            named[f"requant_a_kernel|{tag}"] = dict(
                kernel="requant_a_kernel", grid=math.ceil(m * k // 8 / 512) * 256,
                workload=f"activation requant {m}x{k} ({tag})", alg=m * k * 25 // 8)
    return named


def decode_named():
    """The decode launches of `bench.py --only decode`, per case (m rows padded
    to 1, 2, 4 or 8): the default GEMV, the path-invariant GEMV and the W4A16
    GEMV, with the launch shapes their plans give at N = 14336, K = 4096 and
    N = 4096, K = 14336, and their algorithmic bytes per launch."""
    sys.path.insert(0, ROOT)
    from block_scaled_precision_requant_amd import inputs
    relay = {1: ("1, 6, 3, 3", 448), 2: ("2, 8, 2, 2", 576), 4: ("4, 7, 2, 2", 512), 8: ("8, 4, 2, 2", 384)}
    w4_threads_wide = {1: 512, 2: 512, 4: 256, 8: 192}
    named = {}
    for p in inputs.workload("decode").projections:
        m, n, k = p.m, p.n, p.k
        rows = 1 if m <= 1 else 2 if m <= 2 else 4 if m <= 4 else 8
        wide = n > 4096
        int8_alg = n * k * 9 // 8 + m * k * 9 // 8 + 2 * m * n
        named[f"gemv|{p.name}"] = dict(
            kernel=f"gemv_stream_kernel<{rows}, 2, false>", grid=896 * 128 if wide else 256 * 512,
            workload=f"decode GEMV {m}x{n}x{k}", alg=int8_alg)
        if wide:
            named[f"invariant|{p.name}"] = dict(
                kernel=f"gemv_stream_kernel<{rows}, 4, false>", grid=896 * 64,
                workload=f"path-invariant GEMV {m}x{n}x{k}", alg=int8_alg)
        else:
            tmpl, threads = relay[rows]
            named[f"invariant|{p.name}"] = dict(
                kernel=f"gemv_chain_relay_kernel<{tmpl}, false>", grid=256 * threads,
                workload=f"path-invariant GEMV {m}x{n}x{k}", alg=int8_alg)
        named[f"w4a16|{p.name}"] = dict(
            kernel=f"w4a16_stream_kernel<{rows}, 2>", grid=896 * w4_threads_wide[rows] if wide else 256 * 512,
            workload=f"W4A16 GEMV {m}x{n}x{k}", alg=n * k * 9 // 16 + 2 * m * k + 2 * m * n)
    return named


def cmd_traffic(args):
    fetch, write = _counter(args.fetch, "FETCH_SIZE"), _counter(args.write, "WRITE_SIZE")
    f_kib, f_scale = _copy_scale(args.fetch_copy, "FETCH_SIZE")
    w_kib, w_scale = _copy_scale(args.write_copy, "WRITE_SIZE")
    named = json.loads(args.named) if args.named else decode_named() if args.set == "decode" else default_named()
    out = {}
    rows = []
    for label, spec in named.items():
        keys = [k for k in fetch if short_name(k[0]).startswith(spec["kernel"]) and k[1] == spec["grid"]]
        if not keys:
            print(f"no dispatches for {label}", file=sys.stderr)
            continue
        fv = [x for k in keys for x in fetch[k]]
        wv = [x for k in keys if k in write for x in write[k]]
        fk, wk = sum(fv) / len(fv), (sum(wv) / len(wv) if wv else float("nan"))
        total = fk * 1024 * f_scale + wk * 1024 * w_scale
        fam = family(keys[0][0])
        out[label] = dict(kernel=short_name(keys[0][0]), workload=spec["workload"], grid_work_items=spec["grid"],
                          source_digest=source_digest(SOURCES[fam]) if fam else None, dispatches=len(fv),
                          fetch_size_kib_per_launch=fk, write_size_kib_per_launch=wk, fetch_scale=f_scale,
                          write_scale=w_scale, bytes_per_launch=int(round(total)),
                          algorithmic_bytes_per_launch=int(spec["alg"]))
        rows.append(f"| `{short_name(keys[0][0])}` | {spec['workload']} | {len(fv)} | {fk:.1f} | {wk:.1f} | "
                    f"{total / 1e6:.2f} | {spec['alg'] / 1e6:.2f} | {total / spec['alg']:.2f} |")
    with open(args.out_json, "w") as f:
        json.dump(out, f, indent=1)
    lines = ["# HBM traffic per kernel launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (from /tmp, one MI355X, each counter in its own pass):", "", "```"] + args.command + [
             "```", "",
             "Calibration: `bench.py --only copy` runs five 256 MiB device copies, each reading and writing 262144 KiB.",
             "", "| counter | copy reading (KiB / dispatch) | scale to true bytes |", "|---|---|---|",
             f"| FETCH_SIZE | {f_kib:.1f} | x {f_scale:.3f} |", f"| WRITE_SIZE | {w_kib:.1f} | x {w_scale:.3f} |", "",
             "Per launch (counter readings averaged over the dispatches of that launch shape):", "",
             "| kernel | workload | dispatches | FETCH KiB | WRITE KiB | scaled MB / launch | algorithmic MB | ratio |",
             "|---|---|---|---|---|---|---|---|"] + rows
    with open(args.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(args.out_json, args.out_md)


def cmd_sq(args):
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))  # counter -> pass -> dispatch -> value
    for i, d in enumerate(args.dirs):
        for row in _rows(d, "counter_collection.csv"):
            if not short_name(row["Kernel_Name"]).startswith(args.kernel):
                continue
            if _grid(row)[0] != args.grid:
                continue
            per[row["Counter_Name"]][i][int(row.get("Dispatch_Id") or 0)] += float(row["Counter_Value"])
    if not per:
        sys.exit("no matching dispatches")
    lines = [f"# SQ counters: {args.title}", "", f"Kernel `{args.kernel}`, grid {args.grid} work-items; values per",
             "launch summed over the chip, mean over the second half of the dispatches of each pass.", "",
             "Commands (from /tmp, one MI355X):", "", "```"] + args.command + ["```", "",
             "| counter | dispatches used | per launch | per SIMD (1024 SIMDs) |", "|---|---|---|---|"]
    for name in sorted(per):
        # per pass: the dispatches in order (rows of one dispatch summed), second half kept
        half = []
        for passes in per[name].values():
            vals = [passes[k] for k in sorted(passes)]
            half += vals[len(vals) // 2:] or vals
        mean = sum(half) / len(half)
        lines.append(f"| {name} | {len(half)} | {mean:,.0f} | {mean / 1024:,.1f} |")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(args.out)


def main():
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="default benchmark run")
    c = sub.add_parser("traffic")
    for a in ("fetch", "write", "fetch_copy", "write_copy", "out_json", "out_md"):
        c.add_argument(a)
    c.add_argument("--named", help="JSON {label: {kernel, grid, workload, alg}} (default: the --set launches)")
    c.add_argument("--set", choices=["prefill", "decode"], default="prefill",
                   help="launches to summarize: the prefill kernels or the decode GEMVs")
    c.add_argument("--command", action="append", required=True)
    s = sub.add_parser("sq")
    s.add_argument("dirs", nargs="+")
    s.add_argument("--out", required=True)
    s.add_argument("--kernel", required=True)
    s.add_argument("--grid", type=int, required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", action="append", required=True)
    args = p.parse_args()
    {"trace": cmd_trace, "traffic": cmd_traffic, "sq": cmd_sq}[args.cmd](args)


if __name__ == "__main__":
    main()
