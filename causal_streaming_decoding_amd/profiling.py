"""Summaries of rocprofv3 runs of bench.py: kernel times and calibrated HBM bytes.

Three runs of the same bench command feed it:

* a kernel trace (``rocprofv3 --kernel-trace --stats --output-format csv``),
* a ``FETCH_SIZE`` counter pass and a ``WRITE_SIZE`` counter pass
  (``rocprofv3 --pmc ... --output-format csv``), each with ``--calibrate-copy``
  so that the run ends with one 1 GiB device-to-device copy.

The counters report KiB per dispatch in units that need not be bytes moved:
each is scaled by what it reads for the calibration copy, whose true traffic
is 1 GiB read and 1 GiB written. The window-attention record it writes holds a
hash of the kernel's source files, so that a later reader can tell whether the
counters still describe the kernel that is built.

Usage (the second form summarises ``bench.py --all-configs``, the third
``bench.py --lm-head``)::

    python -m causal_streaming_decoding_amd.profiling configs --configs-jsonl <file> \\
        --trace <workload>=<dir> [--trace ...] --out-md profiles/<name>.md
    python -m causal_streaming_decoding_amd.profiling \\
        --trace <out>/prof_trace --fetch <out>/prof_fetch \\
        --write <out>/prof_write --bench-json <out>/prof_bench.json \\
        --steps 256 --out-md profiles/<name>.md --out-traffic profiles/<name>_traffic.txt
    python -m causal_streaming_decoding_amd.profiling lmhead --bench-jsonl <file> \\
        --trace <dir> --fetch <dir> --write <dir> --out-md profiles/<name>.md
"""

import argparse
import csv
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ATTN_SOURCES = ("csrc/attn.hip", "csrc/attn_combine.hpp", "csrc/attn_device.hpp", "csrc/common.hpp",
                "csrc/entropy_ops.hpp")
ATTN_KERNEL = "k_window_attn_bf16"
CALIBRATION_KIB = 1 << 20  # the 1 GiB copy, read once and written once


def attn_source_hash():
    """sha256 over the window-attention kernel's source files, in a fixed order."""
    h = hashlib.sha256()
    for rel in ATTN_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def short_name(name):
    """'void wedlm::k_window_attn_bf16<4>(wedlm::AttnArgs)' -> 'wedlm::k_window_attn_bf16<4>'."""
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def kernel_stats(trace_dir, prefix="wedlm::"):
    """[(kernel, calls, avg_us, min_us, max_us)] for the library's kernels, by total time."""
    out = []
    with open(os.path.join(trace_dir, "run_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            n = short_name(r["Name"])
            if n.startswith(prefix):
                out.append((n, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                            float(r["TotalDurationNs"])))
    out.sort(key=lambda t: -t[5])
    return [t[:5] for t in out]


def counter_values(pmc_dir, counter):
    """({kernel: [KiB per dispatch in dispatch order]}, calibration-copy KiB)."""
    per = {}
    calib = None
    with open(os.path.join(pmc_dir, "run_counter_collection.csv")) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        n = short_name(r["Kernel_Name"])
        v = float(r["Counter_Value"])
        if "copyBuffer" in n:
            calib = v if calib is None else max(calib, v)  # the 1 GiB copy is the largest
            continue
        per.setdefault(n, []).append(v)
    return per, calib


def _bench_line(path):
    with open(path) as f:
        return json.loads([ln for ln in f if ln.startswith("{")][-1])


def summarize(trace, fetch, write, bench_json, steps, out_md, out_traffic, command_trace,
              command_fetch, command_write, counter_bench_json=None):
    """counter_bench_json: the bench line of the counter runs, when they ran
    fewer steps than the traced command (its algorithmic bytes per launch
    then go with the counted bytes; the trace's line still gives the timed
    launch duration)."""
    stats = kernel_stats(trace)
    fetch_kib, fetch_cal = counter_values(fetch, "FETCH_SIZE")
    write_kib, write_cal = counter_values(write, "WRITE_SIZE")
    if fetch_cal is None or write_cal is None:
        raise SystemExit("no calibration copy in the counter runs (bench.py --calibrate-copy)")
    f_fac = fetch_cal / CALIBRATION_KIB
    w_fac = write_cal / CALIBRATION_KIB
    bench = _bench_line(bench_json)
    roof = bench["roofline"]
    croof = _bench_line(counter_bench_json)["roofline"] if counter_bench_json else roof

    def per_launch(d, name, fac):
        vals = d.get(name, [])[-steps:]  # the timed steps are the last dispatches
        return (sum(vals) / len(vals)) * 1024.0 / fac if vals else None

    attn = next(n for n, *_ in stats if ATTN_KERNEL in n)
    a_fetch = per_launch(fetch_kib, attn, f_fac)
    a_write = per_launch(write_kib, attn, w_fac)
    # the counters cover every timed launch; the events a uniform sample of them
    alg = croof.get("algorithmic_bytes_per_launch_all_steps", croof["algorithmic_bytes_per_launch"])
    trace_avg = next(t[2] for t in stats if t[0] == attn)

    lines = [f"# Window step kernels: {bench['config']['workload']}", "",
             "MI355X (gfx950). Durations in microseconds; bytes are per dispatch, averaged over "
             f"the last {steps} dispatches of each kernel (the timed steps). In the commands, "
             "`<repo>` is the repository root.", "",
             "## Kernel trace", "", "```", command_trace, "```", "",
             "| kernel | calls | avg | min | max |", "|---|---|---|---|---|"]
    for n, c, avg, mn, mx in stats:
        lines.append(f"| `{n}` | {c} | {avg:.2f} | {mn:.2f} | {mx:.2f} |")
    lines += ["", f"Bench line of the same command: {bench['value']:.1f} window-steps/s; HIP-event "
              f"average of the attention launch {roof['avg_launch_ms'] * 1e3:.2f} us against "
              f"{trace_avg:.2f} us in the trace "
              f"({abs(roof['avg_launch_ms'] * 1e3 - trace_avg) / trace_avg * 100:.1f} % apart).", "",
              "## HBM byte counters", "", "```", command_fetch, command_write, "```", "",
              f"Calibration (1 GiB copy, read and written once): FETCH_SIZE {fetch_cal:.1f} KiB "
              f"(factor {f_fac:.4f}), WRITE_SIZE {write_cal:.1f} KiB (factor {w_fac:.4f}). Bytes "
              "below are counter / factor.", "",
              "| kernel | read MB / dispatch | written MB / dispatch |", "|---|---|---|"]
    for n, *_ in stats:
        r = per_launch(fetch_kib, n, f_fac)
        w = per_launch(write_kib, n, w_fac)
        if r is None or w is None:
            continue
        lines.append(f"| `{n}` | {r / 1e6:.2f} | {w / 1e6:.2f} |")
    what = ("KV prefix, window q/k/v and the step's logits (the launch carries the entropy "
            "chunk pass) read, output and committed rows written") if "entropy" in roof.get(
                "kernel", "") else "KV prefix + window q/k/v read, output and committed rows written"
    lines += ["", f"Window attention: algorithmic {alg / 1e6:.1f} MB per launch ({what}); counted "
              f"{(a_fetch + a_write) / 1e6:.1f} MB ({(a_fetch + a_write) / alg:.3f} x)."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(out_traffic, "w") as f:
        f.write(f"kernel: {attn}\n")
        f.write(f"source_sha256: {attn_source_hash()}\n")
        f.write(f"workload: {bench['config']['workload']}\n")
        f.write(f"steps: {steps}\n")
        f.write(f"fetch_bytes_per_launch: {a_fetch:.0f}\n")
        f.write(f"write_bytes_per_launch: {a_write:.0f}\n")
        f.write(f"algorithmic_bytes_per_launch: {alg:.0f}\n")
        f.write(f"counted_over_algorithmic: {(a_fetch + a_write) / alg:.4f}\n")
        f.write(f"fetch_factor: {f_fac:.6f}\n")
        f.write(f"write_factor: {w_fac:.6f}\n")
        f.write(f"command_fetch: {command_fetch}\n")
        f.write(f"command_write: {command_write}\n")


def summarize_configs(configs_jsonl, traces, out_md, command_bench, command_trace):
    """Single-step latencies of the other workloads (bench.py --all-configs) and,
    per workload, the kernel durations of a traced run of that workload alone
    (``traces``: [(workload, trace dir)]; ``command_trace`` may hold a
    ``{workload}`` placeholder)."""
    import statistics

    rows = [json.loads(ln) for ln in open(configs_jsonl) if ln.startswith("{")]
    lines = ["# Single-step latencies of the parity workloads", "",
             "MI355X (gfx950). Each timed step starts from the same state and follows a 512 MB "
             "read that evicts the caches; times in microseconds (median, p10, p90 over the timed "
             "steps). *graph*: the step captured once as a HIP graph and replayed between two "
             "timing events (nothing else between its kernels); *eager*: the same launches as one "
             "host call each; *chained*: eagerly, the window already reordered by the previous "
             "step's tail, as in a decoding loop (the cold step runs the reorder first); bf16 "
             "runs the entropy chunk pass in the attention's launch and a split attention's "
             "merge in the tail's launch, the chunk pass also "
             "timed as a launch of its own and on a second stream beside the attention. The "
             "attention and entropy + tail segments come from an eager pass "
             "with timing events between the kernels (each record idles the GPU a few "
             "microseconds: upper bounds); HBM rates are algorithmic bytes over those medians. "
             "H: slot entropies in nats (min / median), and the mask slots whose score clears the "
             "threshold. In the commands, `<repo>` is the repository root.", "",
             "```", command_bench, "```", "",
             "| workload | graph step median | p10 | p90 | eager step | chained step | eager, "
             "entropy pass own launch | eager, entropy pass on a second stream | attention segment "
             "| entropy + tail segment | step GB/s | attention GB/s | H min / median | mask slots "
             "below tau |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        h = r["entropy_histogram"]
        chained = (f"{r['chained_step_us']['median']:.1f}" if "chained_step_us" in r else "-")
        lines.append(
            f"| `{r['workload']}` | {r['step_us']['median']:.1f} | {r['step_us']['p10']:.1f} | "
            f"{r['step_us']['p90']:.1f} | {r['eager_step_us']['median']:.1f} | {chained} | "
            f"{r['eager_separate_entropy_step_us']['median']:.1f} | "
            f"{r['overlap_step_us']['median']:.1f} | "
            f"{r['attn_segment_us']['median']:.1f} | {r['entropy_tail_segment_us']['median']:.1f} | "
            f"{r['step_hbm_gbps_at_median']:.0f} | {r['attn_hbm_gbps_at_segment_median']:.0f} | "
            f"{h['min']:.2f} / {h['median']:.2f} | "
            f"{h['mask_slots_below_tau']} of {h['mask_slots']} |")
    lines += ["", "Entropy histograms (unit bins, nats): "]
    for r in rows:
        h = r["entropy_histogram"]
        nz = [f"{b} {c}" for b, c in zip(h["bins"], h["counts"]) if c]
        lines.append(f"* `{r['workload']}`: " + ", ".join(nz))
    lines += ["", "## Kernel durations per workload", "", "```", command_trace, "```"]
    for workload, trace_dir in traces:
        per = {}
        with open(os.path.join(trace_dir, "run_kernel_trace.csv")) as f:
            for r in csv.DictReader(f):
                n = short_name(r["Kernel_Name"])
                if not n.startswith("wedlm::"):
                    continue
                key = (n, int(r["Grid_Size_X"]) // max(int(r["Workgroup_Size_X"]), 1),
                       int(r["Grid_Size_Y"]), int(r["Workgroup_Size_X"]))
                per.setdefault(key, []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines += ["", f"`{workload}`", "", "| kernel | blocks x rows | threads | launches | median us |",
                  "|---|---|---|---|---|"]
        for (n, gx, gy, wg), v in sorted(per.items(), key=lambda kv: -statistics.median(kv[1])):
            lines.append(f"| `{n}` | {gx} x {gy} | {wg} | {len(v)} | {statistics.median(v):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_counters(csv_paths, out_md, title, intro, commands, xcds=8, cus=256, simds=4,
                       clock_ghz=2.4, mfma_per_wave_page=12, unit="16-key page"):
    """SQ / GRBM counter passes of a kernel, one column per launch (kernel
    instantiation and workgroups), medians over the dispatches, and the ratios
    read from them: MFMA busy, instruction mix per MFMA, LDS bank conflicts,
    waits.

    ``csv_paths``: run_counter_collection.csv of each pass (counters summed
    over the chip by rocprofv3, GRBM_GUI_ACTIVE over the XCDs)."""
    import collections
    import statistics

    per_shape = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in csv_paths:
        per_dispatch = collections.defaultdict(dict)
        shape = {}
        for r in csv.DictReader(open(path)):
            d = r["Dispatch_Id"]
            per_dispatch[d][r["Counter_Name"]] = float(r["Counter_Value"])
            wgs = int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1)
            shape[d] = (short_name(r["Kernel_Name"]).replace("wedlm::", ""), wgs)
        for d, vals in per_dispatch.items():
            for k, v in vals.items():
                per_shape[shape[d]][k].append(v)
    shapes = sorted(per_shape)
    med = {w: {k: statistics.median(v) for k, v in per_shape[w].items()} for w in shapes}
    names = sorted({k for w in shapes for k in med[w]})
    lines = [f"# {title}", "", intro, "", "```"] + list(commands) + ["```", "",
             "| counter | " + " | ".join(f"`{w[0]}`, {w[1]} workgroups" for w in shapes) + " |",
             "|---|" + "---|" * len(shapes)]
    for k in names:
        lines.append(f"| `{k}` | " + " | ".join(
            f"{med[w][k]:.4g}" if k in med[w] else "-" for w in shapes) + " |")
    lines += ["", "Derived, per launch shape:", ""]
    for w in shapes:
        m = med[w]
        need = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
                "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU_TRANS_F32")
        if any(k not in m for k in need):
            continue
        active = m["GRBM_GUI_ACTIVE"] / xcds
        mf = m["SQ_INSTS_MFMA"]
        lines.append(
            f"* `{w[0]}`, {w[1]} workgroups: GPU-active {active / (clock_ghz * 1e3):.1f} us per dispatch; MFMA "
            f"busy {100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (active * cus * simds):.1f} % "
            f"(MFMA-busy cycles / (active cycles x {cus} CUs x {simds} SIMDs)); per MFMA "
            f"instruction {m['SQ_INSTS_VALU'] / mf:.2f} VALU (of them "
            f"{m['SQ_INSTS_VALU_TRANS_F32'] / mf:.2f} transcendental), "
            f"{m['SQ_INSTS_SALU'] / mf:.2f} SALU, {m['SQ_INSTS_LDS'] / mf:.2f} LDS, i.e. per "
            f"wavefront and {unit} ({mfma_per_wave_page} MFMAs) "
            f"{mfma_per_wave_page * m['SQ_INSTS_VALU'] / mf:.0f} VALU, "
            f"{mfma_per_wave_page * m['SQ_INSTS_SALU'] / mf:.0f} SALU, "
            f"{mfma_per_wave_page * m['SQ_INSTS_LDS'] / mf:.0f} LDS; LDS bank conflicts "
            f"{100 * m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:.1f} % of LDS-active "
            f"cycles; wave cycles waiting on a dependency "
            f"{100 * m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.1f} %, issuing "
            f"{100 * m['SQ_ACTIVE_INST_ANY'] / m['SQ_WAVE_CYCLES']:.1f} %.")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in m and "SQ_WAIT_ANY" in m:
            lines.append(
                f"  `{w[0]}`, {w[1]} workgroups: of the MFMA-busy cycles, "
                f"{100 * m['SQ_VALU_MFMA_COEXEC_CYCLES'] / m['SQ_VALU_MFMA_BUSY_CYCLES']:.1f} % have "
                f"a VALU instruction executing beside them; wave cycles waiting on anything "
                f"(counters, barriers, dependencies) {100 * m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.1f} %.")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _dispatch_runs(csv_path, name_prefix, value_key, counter=None):
    """Runs of consecutive dispatches of one kernel with the same (name, grid),
    in dispatch order: [(name, grid, [values])]."""
    with open(csv_path) as f:
        rows = list(csv.DictReader(f))
    if counter is not None:
        rows = [r for r in rows if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    runs = []
    for r in rows:
        n = short_name(r["Kernel_Name"])
        if not n.startswith(name_prefix):
            continue
        key = (n, int(r["Grid_Size"]) if "Grid_Size" in r else int(r["Grid_Size_X"]))
        v = value_key(r)
        if runs and runs[-1][0] == key:
            runs[-1][1].append(v)
        else:
            runs.append((key, [v]))
    return [(k[0], k[1], v) for k, v in runs]


def summarize_lm_head(bench_jsonl, trace, fetch, write, out_md, command_bench, command_trace,
                      command_fetch, command_write):
    """Vocabulary projection: per shape, the partial-reduction kernel's trace
    duration and calibrated HBM bytes against its algorithmic bytes."""
    import statistics

    lines_in = [json.loads(ln) for ln in open(bench_jsonl) if ln.startswith("{")]
    kern = "wedlm::k_lm_head_partial"
    dur = _dispatch_runs(os.path.join(trace, "run_kernel_trace.csv"), kern,
                         lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    _, f_cal = counter_values(fetch, "FETCH_SIZE")
    _, w_cal = counter_values(write, "WRITE_SIZE")
    f_fac, w_fac = f_cal / CALIBRATION_KIB, w_cal / CALIBRATION_KIB
    fet = _dispatch_runs(os.path.join(fetch, "run_counter_collection.csv"), kern,
                         lambda r: float(r["Counter_Value"]), "FETCH_SIZE")
    wri = _dispatch_runs(os.path.join(write, "run_counter_collection.csv"), kern,
                         lambda r: float(r["Counter_Value"]), "WRITE_SIZE")
    if not (len(dur) == len(fet) == len(wri) == len(lines_in)):
        raise SystemExit(f"shape runs do not line up: {len(dur)} {len(fet)} {len(wri)} {len(lines_in)}")
    out = ["# Fused vocabulary projection + selection", "",
           "MI355X (gfx950). One row per shape of `bench.py --lm-head`: the bench's HIP-event "
           "median of the whole call (projection kernel, partial merge, selection), the trace "
           "median of the projection kernel `k_lm_head_partial` alone, and that kernel's HBM "
           "bytes from the counters (calibrated by a 1 GiB copy, mean over the timed calls). "
           "In the commands, `<repo>` is the repository root.", "",
           "```", command_bench, command_trace, command_fetch, command_write, "```", "",
           f"Calibration: FETCH_SIZE factor {f_fac:.4f}, WRITE_SIZE factor {w_fac:.4f}.", "",
           "| shape | rows x hidden x V | call median us | kernel | kernel median us | "
           "algorithmic MB | read MB | written MB | counted / algorithmic | roofline |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for ln, (name, grid, d), (_, _, fv), (_, _, wv) in zip(lines_in, dur, fet, wri):
        # the kernel's first template argument is its 32-row blocks per workgroup
        rb = int(name.split("<", 1)[1].split(",", 1)[0])
        groups = -(-ln["rows"] // (32 * rb))
        rd = statistics.mean(fv[-ln["steps"]:]) * 1024.0 / f_fac
        wr = statistics.mean(wv[-ln["steps"]:]) * 1024.0 / w_fac
        alg = ln["algorithmic_bytes"]
        roof = ln["roofline"]
        out.append(
            f"| `{ln['workload']}` | {ln['rows']} x {ln['hidden']} x {ln['V']} | "
            f"{ln['us']['median']:.1f} | `{name}` ({groups} row groups) | "
            f"{statistics.median(d[-ln['steps']:]):.1f} | {alg / 1e6:.1f} | {rd / 1e6:.1f} | "
            f"{wr / 1e6:.2f} | {(rd + wr) / alg:.3f} | {roof['bound']} {roof['frac'] * 100:.1f} % |")
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")


def _entropy_dispatches(trace, fetch, write, grid):
    """Trace durations (us) and FETCH / WRITE KiB of the chunk-pass dispatches
    whose grid has `grid` threads, in dispatch order."""
    kern = "wedlm::k_entropy_partial"
    dur = []
    with open(os.path.join(trace, "run_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            if short_name(r["Kernel_Name"]).startswith(kern) and \
                    int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) == grid:
                dur.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    vals = {}
    for d, counter in ((fetch, "FETCH_SIZE"), (write, "WRITE_SIZE")):
        with open(os.path.join(d, "run_counter_collection.csv")) as f:
            vals[counter] = [float(r["Counter_Value"]) for r in csv.DictReader(f)
                             if r["Counter_Name"] == counter and int(r["Grid_Size"]) == grid
                             and short_name(r["Kernel_Name"]).startswith(kern)]
    return dur, vals["FETCH_SIZE"], vals["WRITE_SIZE"]


def summarize_entropy(items, out_md, commands, peak_gbps=8000.0):
    """Entropy chunk pass as a launch of its own: per workload, the trace median
    of k_entropy_partial and its calibrated HBM bytes against the logits.

    items: [(workload, rows, V, element bytes, trace dir, fetch dir, write dir)];
    the fetch and write runs include the 1 GiB calibration copy."""
    import statistics

    out = ["# Entropy chunk pass (`k_entropy_partial`) as a launch of its own", "",
           "MI355X (gfx950). For each workload, every launch of the full-vocabulary chunk pass "
           "that runs as its own kernel (the ragged g = 7 step's default; the other single-step "
           "workloads' `eager, entropy pass own launch` column; the streaming loop with "
           "`--separate-entropy`): the trace median of the kernel, the logits it must read "
           "(rows x V x element size, the algorithmic bytes; the partials it writes are "
           "16 bytes per chunk and row), and the HBM bytes counted by `FETCH_SIZE` and "
           "`WRITE_SIZE` (KiB per dispatch, calibrated by a 1 GiB device copy, mean over the "
           "dispatches). In the commands, `<repo>` is the repository root.", "",
           "```", *commands, "```", "",
           "| workload | rows x V | chunk blocks | launches | kernel median us | logits MB | "
           "read MB | written KB | read / logits | logits TB/s | % of 8 TB/s |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name, rows, V, elt, trace, fetch, write in items:
        chunk = 256 * 8 * (16 // elt)
        chunks = -(-V // chunk)
        grid = chunks * 256 * rows
        dur, fv, wv = _entropy_dispatches(trace, fetch, write, grid)
        _, f_cal = counter_values(fetch, "FETCH_SIZE")
        _, w_cal = counter_values(write, "WRITE_SIZE")
        if not dur or not fv or not wv or f_cal is None or w_cal is None:
            out.append(f"| `{name}` | {rows} x {V} | {chunks} x {rows} | 0 | - | - | - | - | - | - | - |")
            continue
        f_fac, w_fac = f_cal / CALIBRATION_KIB, w_cal / CALIBRATION_KIB
        med = statistics.median(dur)
        logits = rows * V * elt
        rd = statistics.mean(fv) * 1024.0 / f_fac
        wr = statistics.mean(wv) * 1024.0 / w_fac
        tbs = logits / (med * 1e-6) / 1e12
        out.append(f"| `{name}` | {rows} x {V} | {chunks} x {rows} | {len(dur)} | {med:.2f} | "
                   f"{logits / 1e6:.1f} | {rd / 1e6:.1f} | {wr / 1e3:.1f} | {rd / logits:.3f} | "
                   f"{tbs:.2f} | {100 * tbs * 1e3 / peak_gbps:.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(out) + "\n")


def read_traffic(path, workload):
    """Counted HBM bytes over algorithmic bytes of the attention launch, or None
    when the record does not apply.

    The ratio, not a byte count, is what carries over between runs of
    different lengths (the prefix, hence the bytes per launch, grows with the
    steps). The record applies only to the same workload and to the kernel
    source it was measured on.
    """
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for ln in f:
            if ": " in ln:
                k, v = ln.rstrip("\n").split(": ", 1)
                rec[k] = v
    if rec.get("source_sha256") != attn_source_hash() or rec.get("workload") != workload:
        return None
    counted = float(rec["fetch_bytes_per_launch"]) + float(rec["write_bytes_per_launch"])
    return counted / float(rec["algorithmic_bytes_per_launch"])


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "lmhead":
        ap = argparse.ArgumentParser()
        ap.add_argument("mode")
        ap.add_argument("--bench-jsonl", required=True)
        ap.add_argument("--trace", required=True)
        ap.add_argument("--fetch", required=True)
        ap.add_argument("--write", required=True)
        ap.add_argument("--out-md", required=True)
        for k in ("bench", "trace", "fetch", "write"):
            ap.add_argument(f"--command-{k}", default="")
        a = ap.parse_args()
        summarize_lm_head(a.bench_jsonl, a.trace, a.fetch, a.write, a.out_md, a.command_bench,
                          a.command_trace, a.command_fetch, a.command_write)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        ap = argparse.ArgumentParser()
        ap.add_argument("mode")
        ap.add_argument("--csv", action="append", required=True)
        ap.add_argument("--out-md", required=True)
        ap.add_argument("--title", required=True)
        ap.add_argument("--intro", default="")
        ap.add_argument("--command", action="append", default=[])
        ap.add_argument("--mfma-per-wave-page", type=int, default=12,
                        help="MFMA instructions per wavefront and work unit of the kernel")
        ap.add_argument("--unit", default="16-key page", help="the work unit's name")
        a = ap.parse_args()
        summarize_counters(a.csv, a.out_md, a.title, a.intro, a.command,
                           mfma_per_wave_page=a.mfma_per_wave_page, unit=a.unit)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "entropy":
        ap = argparse.ArgumentParser()
        ap.add_argument("mode")
        ap.add_argument("--configs-jsonl", required=True)
        ap.add_argument("--trace", required=True)
        ap.add_argument("--fetch", required=True)
        ap.add_argument("--write", required=True)
        ap.add_argument("--stream-json", default=None)
        ap.add_argument("--stream-trace", default=None)
        ap.add_argument("--stream-fetch", default=None)
        ap.add_argument("--stream-write", default=None)
        ap.add_argument("--out-md", required=True)
        ap.add_argument("--command", action="append", default=[])
        a = ap.parse_args()
        items = []
        for ln in open(a.configs_jsonl):
            if ln.startswith("{"):
                d = json.loads(ln)
                elt = 4 if d["dtype"] == "f32" else 2
                items.append((d["workload"], d["rows"], d["vocab"], elt, a.trace, a.fetch, a.write))
        if a.stream_json:
            d = _bench_line(a.stream_json)
            c = d["config"]
            items.append((c["workload"] + " (--separate-entropy)", c["batch"] * c["window"],
                          c["vocab"], 2, a.stream_trace, a.stream_fetch, a.stream_write))
        summarize_entropy(items, a.out_md, a.command)
        return
    if len(sys.argv) > 1 and sys.argv[1] == "configs":
        ap = argparse.ArgumentParser()
        ap.add_argument("mode")
        ap.add_argument("--configs-jsonl", required=True)
        ap.add_argument("--trace", action="append", required=True,
                        help="WORKLOAD=DIR, one per workload traced alone")
        ap.add_argument("--out-md", required=True)
        ap.add_argument("--command-bench", default="")
        ap.add_argument("--command-trace", default="")
        a = ap.parse_args()
        traces = [tuple(t.split("=", 1)) for t in a.trace]
        summarize_configs(a.configs_jsonl, traces, a.out_md, a.command_bench, a.command_trace)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--bench-json", required=True)
    ap.add_argument("--counter-bench-json", default=None)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--out-md", required=True)
    ap.add_argument("--out-traffic", required=True)
    ap.add_argument("--command-trace", default="")
    ap.add_argument("--command-fetch", default="")
    ap.add_argument("--command-write", default="")
    a = ap.parse_args()
    summarize(a.trace, a.fetch, a.write, a.bench_json, a.steps, a.out_md, a.out_traffic,
              a.command_trace, a.command_fetch, a.command_write, a.counter_bench_json)


if __name__ == "__main__":
    main()
