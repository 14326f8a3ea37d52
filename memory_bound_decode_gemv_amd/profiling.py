"""Summaries of rocprofv3 runs for the profiles/ directory (host-side, reads CSVs).

Counters: two `rocprofv3 --pmc` runs (FETCH_SIZE, then WRITE_SIZE) of
`bench.py --profile-kernels`, which launches each kernel eagerly on a known
workload next to a plain 1 GiB device-to-device copy.  The copy's counters
calibrate the others: on MI355X FETCH_SIZE reads half the bytes a kernel
fetches while WRITE_SIZE reads them exactly, so each counter is scaled by
(bytes the copy moved) / (what the counter read for it).  The HBM traffic per
launch of a kernel is then
    FETCH_SIZE * fetch_scale + WRITE_SIZE * write_scale     (KiB * 1024).
Each entry records a hash of the kernel's source files; bench.py reports the
traffic only while that hash still matches the tree.

Why FETCH_SIZE reads half: for gfx950 rocprofiler-sdk derives it as
    (TCC_BUBBLE*128 + (TCC_EA0_RDREQ - TCC_BUBBLE - TCC_EA0_RDREQ_32B)*64
     + TCC_EA0_RDREQ_32B*32) / 1024,
i.e. it takes TCC_BUBBLE to count the 128-byte read requests.  On MI355X
TCC_BUBBLE reads 0 while every L2-to-memory read request carries 128 bytes
(TCC_EA0_RDREQ of a 1 GiB streaming read is 2^30 / 128 plus a few hundred,
TCC_EA0_RDREQ_32B is 0), so each request is counted as 64 bytes.  Two more
passes (--tcc) record those request counters and the L2 tag counters
(TCC_REQ, TCC_READ, TCC_HIT, TCC_MISS); 128 * TCC_EA0_RDREQ is then a second
estimate of the bytes read from memory that needs no calibration.

    python -m memory_bound_decode_gemv_amd.profiling counters FETCH.csv WRITE.csv [--tcc TCCA.csv TCCB.csv]
    python -m memory_bound_decode_gemv_amd.profiling trace KERNEL_STATS.csv [--runs KERNEL_TRACE.csv] --md OUT.md
    python -m memory_bound_decode_gemv_amd.profiling suite SUITE.jsonl --md OUT.md
    python -m memory_bound_decode_gemv_amd.profiling suite A.jsonl B.jsonl --condense --filter RE --md OUT.md
    python -m memory_bound_decode_gemv_amd.profiling pmc PASS1.csv PASS2.csv ... --kernels RE --labels L1,L2,.. \
        --per 4 --md OUT.md

pmc: SQ counters of `bench.py --profile-small-m` (several --pmc passes of the
same program): the dispatches of the kernels matching --kernels, in program
order, are grouped --per at a time (one group per label) and each counter is
averaged over a group, with a few derived figures (instructions per wave,
vector-ALU busy share).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PROFILES = os.path.join(ROOT, "profiles")
GIB = 1 << 30

# Profiled kernels: key -> (kernel-name pattern, workload, algorithmic bytes per launch, sources)
KERNELS = {
    "gemv_q4_0_m1_28672x8192": (
        r"k_q4_m1_ldsrow<", "Q4_0 x Q8_1, M = 1, N = 28672, K = 8192",
        18 * 28672 * 8192 // 32 + 36 * 8192 // 32 + 4 * 28672,
        ["gemv_q4_0_m1.hip", "q4_common.h", "q81_rules.h", "dg_device.h", "dg_internal.h"]),
    "gemv_q8_0_m1_28672x8192": (
        r"k_units<[^>]*UnitsQ8_0", "Q8_0 x Q8_1, M = 1, N = 28672, K = 8192",
        34 * 28672 * 8192 // 32 + 36 * 8192 // 32 + 4 * 28672,
        ["gemv_m1_units.hip", "q4_common.h", "dg_device.h", "dg_internal.h"]),
    "gemv_q4_0_m16_4096x14336": (
        r"k_q(mfma|res)<", "Q4_0 x Q8_1, M = 16, N = 4096, K = 14336 (matrix cores)",
        18 * 4096 * 14336 // 32 + 16 * 36 * 14336 // 32 + 4 * 16 * 4096,
        ["gemv_q4_0_mfma.hip", "gemv_qmfma_res.hip", "mfma_formats.h", "q4_common.h", "dg_device.h", "dg_internal.h"]),
    "gemv_f16_4096x4096": (
        r"k_gemv_wide<false", "fp16 GEMV, N = K = 4096",
        2 * 4096 * 4096 + 2 * 4096 + 2 * 4096,
        ["gemv_dense.hip", "dg_device.h"]),
    "gemv_nf4_28672x8192_b64": (
        r"k_nf4_rows<", "NF4 x bf16, M = 1, N = 28672, K = 8192, block 64",
        28672 * 8192 // 2 + 4 * 28672 * (8192 // 64) + 2 * 8192 + 64 + 4 * 28672,
        ["gemv_nf4.hip", "dg_device.h", "dg_internal.h"]),
    "stream_read_1GiB": (
        r"k_stream_read_wave<", "streaming read of 1 GiB", GIB,
        ["stream_read.hip", "dg_device.h"]),
}
CALIBRATION = (r"__amd_rocclr_copyBuffer", GIB)   # the 1 GiB copy: GIB read, GIB written


def sources_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    n = name.replace("dg::(anonymous namespace)::", "")
    return re.sub(r"\((unsigned|float|int|long|void|short)[^)]*\)$", "", n)[:80]


def load_counter_csv(path):
    d = collections.defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            d[(row["Kernel_Name"], row["Counter_Name"])].append(float(row["Counter_Value"]))
    return d


def _values(d, pattern, counter):
    out = []
    for (name, c), v in d.items():
        if c == counter and re.search(pattern, name):
            out.extend(v)
    return out


TCC_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_EA0_RDREQ_DRAM_sum",
                "TCC_REQ_sum", "TCC_READ_sum", "TCC_HIT_sum", "TCC_MISS_sum")


def _tcc_means(tcc, pattern, pick_max=False):
    out = {}
    for ctr in TCC_COUNTERS:
        v = _values(tcc, pattern, ctr)
        if v:
            out[ctr] = max(v) if pick_max else sum(v) / len(v)
    return out


def counters_summary(fetch_csv, write_csv, tcc_csvs=()):
    fetch = load_counter_csv(fetch_csv)
    write = load_counter_csv(write_csv)
    cal_pat, cal_bytes = CALIBRATION
    cal_f = max(_values(fetch, cal_pat, "FETCH_SIZE"))
    cal_w = max(_values(write, cal_pat, "WRITE_SIZE"))
    fs = cal_bytes / (cal_f * 1024)
    ws = cal_bytes / (cal_w * 1024)
    tcc = {}
    for path in tcc_csvs:
        tcc.update(load_counter_csv(path))
    out = {"calibration": {"kernel": "1 GiB device-to-device copy", "bytes": cal_bytes,
                           "fetch_kib": cal_f, "write_kib": cal_w,
                           "fetch_scale": round(fs, 5), "write_scale": round(ws, 5)}}
    if tcc:
        out["calibration"]["tcc"] = {k: round(v, 1) for k, v in _tcc_means(tcc, cal_pat, pick_max=True).items()}
    for key, (pat, what, alg, files) in KERNELS.items():
        fv = _values(fetch, pat, "FETCH_SIZE")
        wv = _values(write, pat, "WRITE_SIZE")
        if not fv or not wv:
            continue
        f_kib = sum(fv) / len(fv)
        w_kib = sum(wv) / len(wv)
        traffic = int(round((f_kib * fs + w_kib * ws) * 1024))
        out[key] = {"workload": what, "dispatches": len(fv), "fetch_kib": round(f_kib, 2),
                    "write_kib": round(w_kib, 2), "hbm_bytes_per_launch": traffic,
                    "algorithmic_bytes_per_launch": alg, "traffic_over_algorithmic": round(traffic / alg, 4),
                    "sources": files, "source_sha256_16": sources_hash(files)}
        t = _tcc_means(tcc, pat) if tcc else {}
        if t:
            out[key]["tcc"] = {k: round(v, 1) for k, v in t.items()}
            if "TCC_EA0_RDREQ_sum" in t:
                rd = 128 * t["TCC_EA0_RDREQ_sum"]
                out[key]["read_bytes_128b_requests"] = int(round(rd))
    return out


def counters_markdown(summary, command_fetch, command_write, command_tcc=""):
    lines = ["# HBM traffic per launch from rocprofv3 counters", "",
             "Commands (run from /tmp on an MI355X, repository at $R):", "",
             f"    {command_fetch}", f"    {command_write}"] + \
            [f"    {c}" for c in command_tcc.split(" ;; ") if c] + ["",
             "Calibration: " + json.dumps(summary["calibration"]), "",
             "| kernel | workload | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / launch "
             "| algorithmic bytes | ratio |", "|---|---|---|---|---|---|---|---|"]
    for k, v in summary.items():
        if k == "calibration":
            continue
        lines.append(f"| {k} | {v['workload']} | {v['dispatches']} | {v['fetch_kib']} | {v['write_kib']} | "
                     f"{v['hbm_bytes_per_launch']} | {v['algorithmic_bytes_per_launch']} | "
                     f"{v['traffic_over_algorithmic']} |")
    rows = [(k, v) for k, v in summary.items() if k != "calibration" and v.get("tcc")]
    cal = summary["calibration"].get("tcc")
    if rows or cal:
        lines += ["", "## Why FETCH_SIZE reads half, and a calibration-free cross-check", "",
                  "rocprofiler-sdk derives FETCH_SIZE on gfx950 as (TCC_BUBBLE x 128 + (TCC_EA0_RDREQ - TCC_BUBBLE "
                  "- TCC_EA0_RDREQ_32B) x 64 + TCC_EA0_RDREQ_32B x 32) / 1024 KiB: TCC_BUBBLE is taken to count the "
                  "128-byte read requests.  The passes below show TCC_BUBBLE = 0 and TCC_EA0_RDREQ_32B = 0 for every "
                  "kernel, while TCC_EA0_RDREQ of the 1 GiB streaming read is 2^30 / 128 (8388608) plus a few "
                  "hundred: each L2-to-memory read request moves 128 bytes and the formula counts it as 64.  Hence "
                  "the factor 2 of the calibration.  128 x TCC_EA0_RDREQ estimates the bytes read from memory "
                  "without any calibration; `L2 hit share` is TCC_HIT / (TCC_HIT + TCC_MISS).", "",
                  "| kernel | TCC_EA0_RDREQ | _32B | TCC_BUBBLE | _DRAM | TCC_REQ | TCC_HIT | TCC_MISS | L2 hit share "
                  "| 128 x RDREQ bytes | over algorithmic |", "|---|---|---|---|---|---|---|---|---|---|---|"]
        if cal:
            rows = [("1 GiB copy (calibration)", {"tcc": cal, "algorithmic_bytes_per_launch": GIB})] + rows
        for k, v in rows:
            t = v["tcc"]
            cells = ["" if c not in t else f"{t[c]:.0f}" for c in
                     ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_EA0_RDREQ_DRAM_sum",
                      "TCC_REQ_sum", "TCC_HIT_sum", "TCC_MISS_sum")]
            hm = t.get("TCC_HIT_sum", 0) + t.get("TCC_MISS_sum", 0)
            cells.append(f"{t.get('TCC_HIT_sum', 0) / hm:.3f}" if hm else "")
            if "TCC_EA0_RDREQ_sum" in t:
                rd = 128 * t["TCC_EA0_RDREQ_sum"]
                cells += [f"{rd:.0f}", f"{rd / v['algorithmic_bytes_per_launch']:.4f}"]
            else:
                cells += ["", ""]
            lines.append(f"| {k} | " + " | ".join(cells) + " |")
    return "\n".join(lines) + "\n"


def trace_segments(trace_csv, min_launches=30, idle_us=200.0):
    """Per-kernel runs of launches from a rocprofv3 kernel-trace CSV: a run
    ends where the kernel was idle for more than idle_us (each timed graph of
    a benchmark is one run).  -> {kernel: [(launches, mean us, median us)]}"""
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            if "dg::" in r["Kernel_Name"]:
                rows.append((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort(key=lambda r: r[1])
    out = {}
    for name in sorted({r[0] for r in rows}):
        q = [r for r in rows if r[0] == name]
        runs, cur = [], [q[0]]
        for a, b in zip(q, q[1:]):
            if (b[1] - a[2]) / 1e3 > idle_us:
                runs.append(cur)
                cur = []
            cur.append(b)
        runs.append(cur)
        res = []
        for run in runs:
            if len(run) >= min_launches:
                d = sorted((e - s) / 1e3 for _, s, e in run)
                res.append((len(d), sum(d) / len(d), d[len(d) // 2]))
        if res:
            out[short_name(name)] = res
    return out


def launch_runs(trace_csv, min_launches=30, idle_us=5000.0):
    """Every run of back-to-back launches (any kernel of the library) in
    launch order: a run ends at an idle gap of more than idle_us.  For each:
    kernel, launches, median duration (end - start), median gap (next start -
    this end) and median period (next start - this start), in microseconds."""
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            if "dg::" in r["Kernel_Name"]:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    runs, cur = [], [rows[0]] if rows else []
    for a, b in zip(rows, rows[1:]):
        if (b[0] - a[1]) / 1e3 > idle_us:
            runs.append(cur)
            cur = []
        cur.append(b)
    if cur:
        runs.append(cur)
    out = []
    for run in runs:
        if len(run) < min_launches:
            continue
        med = lambda v: sorted(v)[len(v) // 2]
        dur = [(e - s) / 1e3 for s, e, _ in run]
        gap = [(b[0] - a[1]) / 1e3 for a, b in zip(run, run[1:])]
        per = [(b[0] - a[0]) / 1e3 for a, b in zip(run, run[1:])]
        out.append((short_name(run[0][2]), len(run), med(dur), med(gap), med(per)))
    return out


def launch_cost_markdown(trace_csv, command, labels, nbytes):
    """The runs of a --profile-launch-cost trace, and for each workload that is
    not a plain read the split of its duration into streaming (bytes over the
    rate fitted between the two largest reads), the launch floor (the first
    workload: one wave, one 16-byte load) and the rest (ramp and drain)."""
    runs = launch_runs(trace_csv)
    lines = ["# Per-launch cost of back-to-back launches (rocprofv3 --kernel-trace)", "", "Command:", ""]
    lines += [f"    {c}" for c in command.split(" ;; ")]
    lines += ["",
              "Each row is one graph of back-to-back launches, replayed three times back to back (medians over "
              "every launch of the run).  duration = end - start of a kernel; gap = next start - this end; "
              "period = next start - this start, the time per launch back to back.", "",
              "| workload | bytes per launch | kernel | launches | median duration us | median gap us | "
              "median period us |", "|---|---|---|---|---|---|---|"]
    rows = list(zip(labels, nbytes, runs))
    for lab, nb, (name, n, dur, gap, per) in rows:
        lines.append(f"| {lab} | {nb} | {name} | {n} | {dur:.3f} | {gap:.3f} | {per:.3f} |")
    reads = sorted([(nb, r[2]) for lab, nb, r in rows if lab.startswith("read ")])
    if len(reads) >= 2 and rows:
        (b1, t1), (b2, t2) = reads[-2], reads[-1]
        rate = (b2 - b1) / (t2 - t1) / 1e3   # GB/s
        floor = rows[0][2][2]
        lines += ["", "Under kernel tracing every dispatch carries the profiler's own overhead (the gaps of the "
                  "short kernels); for kernels longer than that the next dispatch is ready before the current one "
                  "ends (gap 0), as in a graph replayed without the profiler.", "",
                  f"Split of each GEMV's duration: streaming = bytes / {rate:.0f} GB/s (the slope between the two "
                  f"largest reads), the launch floor {floor:.3f} us (the shortest kernel that reads memory), and "
                  "the rest (ramp and drain).  No kernel that reads HBM finishes below the floor, so a launch over "
                  "B bytes cannot take less than floor + B / rate.", "",
                  "| workload | streaming us | floor us | rest us | duration us | floor + streaming: best GB/s |",
                  "|---|---|---|---|---|---|"]
        for lab, nb, (name, n, dur, gap, per) in rows[1:]:
            if lab.startswith("read ") or not nb:
                continue
            st = nb / rate / 1e3
            lines.append(f"| {lab} | {st:.2f} | {floor:.2f} | {dur - floor - st:.2f} | {dur:.2f} | "
                         f"{nb / (floor + st) / 1e3:.0f} |")
    return "\n".join(lines) + "\n"


def trace_markdown(stats_csv, command, trace_csv=None):
    lines = ["# Kernel durations from rocprofv3 --kernel-trace --stats", "", "Commands:", ""]
    lines += [f"    {c}" for c in command.split(" ;; ")]
    lines += ["", "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    with open(stats_csv) as f:
        for row in csv.DictReader(f):
            if "dg::" not in row["Name"]:
                continue
            lines.append(f"| {short_name(row['Name'])} | {row['Calls']} | {float(row['AverageNs']) / 1e3:.3f} | "
                         f"{float(row['MinNs']) / 1e3:.3f} | {float(row['MaxNs']) / 1e3:.3f} | "
                         f"{float(row['Percentage']):.2f} |")
    if trace_csv:
        lines += ["", "Runs of back-to-back launches of the GEMV kernels (one per timed graph, in program order; a "
                  "run ends at an idle gap of more than 200 us):", "", "| kernel | launches | mean us | median us |",
                  "|---|---|---|---|"]
        for name, runs in trace_segments(trace_csv).items():
            if "stream_read" in name:
                continue
            for n, mean, med in runs:
                lines.append(f"| {name} | {n} | {mean:.3f} | {med:.3f} |")
    return "\n".join(lines) + "\n"


def suite_markdown(jsonl, command, name_filter=None):
    """A table of `bench.py --suite` records (one JSON object per line)."""
    recs = []
    with open(jsonl) as f:
        for line in f:
            r = json.loads(line)
            if name_filter and not re.search(name_filter, r.get("name", "")):
                continue
            recs.append(r)
    keys = ("name", "us_per_call", "iqr_us", "gbps", "mbu_ceiling", "mbu_spec")
    extra = sorted({k for r in recs for k in r} - set(keys) - {"bytes"})
    lines = ["# bench.py --suite records", "", "Command:", "", f"    {command}", "",
             "| " + " | ".join(keys + tuple(extra)) + " |", "|" + "---|" * (len(keys) + len(extra))]
    for r in recs:
        lines.append("| " + " | ".join(str(r.get(k, "")) for k in keys + tuple(extra)) + " |")
    return "\n".join(lines) + "\n"


_RECORD_KEYS = {"name", "us_per_call", "iqr_us", "bytes", "gbps", "mbu_spec", "mbu_ceiling", "M", "copies",
                "variant", "columns_per_s", "change_vs_prev_M", "note", "cache"}


def _config(r) -> str:
    """The launch configuration a record was timed with, as one short string."""
    parts = [str(r["variant"])] if "variant" in r else []
    parts += [f"{k}={r[k]}" for k in sorted(r) if k not in _RECORD_KEYS]
    for k in ("note", "cache"):
        if k in r:
            parts.append(str(r[k]))
    return " ".join(parts)


def suite_condensed_markdown(jsonls, command, name_filter=None):
    """One line per (workload, M) of `bench.py --suite` records: the library's
    default launch (the record whose variant is "default", else the only one)
    and the fastest configuration the sweep tried, with the run's ceiling."""
    recs, ceilings = [], []
    for path in jsonls:
        file_recs, file_ceil, probe = [], None, None
        with open(path) as f:
            for line in f:
                r = json.loads(line)
                if r.get("name") == "ceiling":
                    # the last ceiling record of a run is its denominator: the probe's best read, or a
                    # kernel's faster demonstrated read when one beat the probe
                    file_ceil = r["gbps"]
                    probe = r.get("probe_gbps", probe if probe is not None else r["gbps"])
                if name_filter and not re.search(name_filter, r.get("name", "")):
                    continue
                if "us_per_call" in r:
                    file_recs.append(r)
        if file_ceil is not None:
            ceilings.append((file_ceil, probe))
            for r in file_recs:
                if r.get("gbps") and r.get("mbu_ceiling") is not None:
                    r = dict(r, mbu_ceiling=round(r["gbps"] / file_ceil, 4))
                recs.append(r)
        else:
            recs.extend(file_recs)
    groups = collections.OrderedDict()
    for r in recs:
        label = " ".join([r["name"]] + [str(r[k]) for k in ("cache", "note") if k in r])
        groups.setdefault((label, r.get("M")), []).append(r)
    lines = ["# bench.py --suite, condensed", "", "Commands:", ""] + [f"    {c}" for c in command.split(" ;; ")]
    lines += ["", "Measured streaming-read ceiling of the run(s): " +
              (", ".join(f"{g:.1f} GB/s" + ("" if p is None or abs(p - g) < 0.05 else
                                          f" (a kernel's demonstrated read; the probe's best {p:.1f} GB/s)")
                         for g, p in ceilings) or "not in these records") + ".",
              "`default` is the launch the library picks by itself; `best` is the fastest configuration the "
              "sweep timed (median of HIP-graph replays, microseconds per call).", "",
              "| workload | M | default us | default GB/s | of ceiling | columns/s | vs previous M | best us | "
              "best configuration | configs timed |", "|---|---|---|---|---|---|---|---|---|---|"]
    for (name, m), rs in groups.items():
        dflt = [r for r in rs if r.get("variant") == "default"]
        d = dflt[0] if dflt else (rs[0] if len(rs) == 1 else None)
        b = min(rs, key=lambda r: r["us_per_call"])
        cells = [name, "" if m is None else str(m)]
        if d is not None:
            chg = d.get("change_vs_prev_M")
            cells += [f"{d['us_per_call']:.3f}", f"{d.get('gbps', 0):.1f}",
                      "" if d.get("mbu_ceiling") is None else f"{d['mbu_ceiling']:.3f}",
                      "" if d.get("columns_per_s") is None else f"{d['columns_per_s']:.0f}",
                      "" if chg is None else f"{chg:+.3f}"]
        else:
            cells += ["", "", "", "", ""]
        cells += [f"{b['us_per_call']:.3f}", _config(b), str(len(rs))]
        lines.append("| " + " | ".join(cells) + " |")
    return "\n".join(lines) + "\n"


def pmc_summary(csvs, kernel_re, labels, per):
    """Per-label averages of every counter in the --pmc CSVs (one CSV per pass)."""
    rows = None
    meta = []
    for path in csvs:
        disp = collections.OrderedDict()
        with open(path) as f:
            for r in csv.DictReader(f):
                if not re.search(kernel_re, r["Kernel_Name"]):
                    continue
                d = disp.setdefault(int(r["Dispatch_Id"]), {"_name": r["Kernel_Name"], "_vgpr": r["VGPR_Count"],
                                                            "_wg": r["Workgroup_Size"], "_grid": r["Grid_Size"],
                                                            "_lds": r["LDS_Block_Size"]})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        seq = [v for _, v in sorted(disp.items())]
        if rows is None:
            rows = [dict(v) for v in seq]
        else:
            for a, b in zip(rows, seq):
                a.update({k: v for k, v in b.items() if not k.startswith("_")})
    out = []
    for i, lab in enumerate(labels):
        grp = rows[i * per:(i + 1) * per]
        if not grp:
            break
        avg = {k: sum(g[k] for g in grp) / len(grp) for k in grp[0] if not k.startswith("_")}
        short = re.sub(r"^void |dg::|\(anonymous namespace\)::|mfma::", "", grp[0]["_name"])
        short = short.split("(")[0]
        out.append({"label": lab, "kernel": short, "vgpr": grp[0]["_vgpr"], "wg": grp[0]["_wg"],
                    "grid_threads": grp[0]["_grid"], "lds": grp[0]["_lds"], **avg})
    return out


def pmc_markdown(summary, command):
    lines = ["# SQ counters of the small-batch Q4_0 GEMV", "", "Command (one run per counter pass):", "",
             f"    {command}", "",
             "Per launch, averaged over four dispatches.  `VALU/wave` and `LDS/wave` are instructions per wave; "
             "`VALU busy` is SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES x waves per SIMD (both counters in units of "
             "four cycles): the share of a SIMD's cycles spent issuing vector instructions.  `rocprof VGPR_Count` "
             "is the profiler's field as printed; on gfx950 it reads half the compiler's register count (60 for a "
             "114-register kernel, 80 for 160: allocation granules of 8 counted as 4), so the register counts "
             "and the occupancy they allow are taken from profiles/kernel_resources.md.", "",
             "| workload | kernel | rocprof VGPR_Count | threads/WG | waves | waves/SIMD | VALU/wave | MFMA | LDS/wave | "
             "LDS bank-conflict cycles | VALU busy |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in summary:
        waves = r.get("SQ_WAVES", 0.0)
        wps = waves / 1024.0
        valu = r.get("SQ_INSTS_VALU", 0.0)
        busy = ""
        if r.get("SQ_WAVE_CYCLES") and r.get("SQ_ACTIVE_INST_VALU"):
            busy = f"{r['SQ_ACTIVE_INST_VALU'] / r['SQ_WAVE_CYCLES'] * min(wps, 8):.2f}"
        lines.append(f"| {r['label']} | `{r['kernel'][:60]}` | {r['vgpr']} | {r['wg']} | {waves:.0f} | {wps:.2f} | "
                     f"{valu / max(waves, 1):.0f} | {r.get('SQ_INSTS_MFMA', 0):.0f} | "
                     f"{r.get('SQ_INSTS_LDS', 0) / max(waves, 1):.0f} | {r.get('SQ_LDS_BANK_CONFLICT', 0):.3g} | "
                     f"{busy} |")
    return "\n".join(lines) + "\n"


_INFO_KEYS = {"TotalNumSgprs": "sgpr", "NumVgprs": "vgpr", "NumAgprs": "agpr", "ScratchSize": "scratch",
              "Occupancy": "occupancy", "LDSByteSize": "lds_static"}


def asm_resources(asm_text):
    """Per kernel of one gfx950 assembly file: the compiler's resource report
    (the "; Kernel info:" block that follows each kernel): VGPRs, AGPRs,
    SGPRs, scratch bytes, statically sized LDS and the waves per SIMD its
    registers allow ("Occupancy"; LDS sized at launch is not counted there)."""
    out = []
    for m in re.finditer(r"; Kernel info:\n((?:;[^\n]*\n)+)", asm_text):
        head = asm_text[:m.start()]
        names = re.findall(r"^\s*\.set\s+(_Z\w+)\.private_seg_size", head, re.M)
        if not names:
            continue
        rec = {"mangled": names[-1]}
        for line in m.group(1).splitlines():
            k, _, v = line[1:].partition(":")
            k = k.strip()
            if k in _INFO_KEYS:
                rec[_INFO_KEYS[k]] = int(re.match(r"\s*(\d+)", v).group(1))
        out.append(rec)
    return out


def _demangle(names):
    import subprocess
    try:
        r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True, check=True)
        return r.stdout.splitlines()
    except (OSError, subprocess.CalledProcessError):
        return list(names)


def resources_markdown(command=""):
    """Compiler resource report of every kernel the library builds, one line
    per kernel template (its instantiations' ranges)."""
    import tempfile
    from . import _build
    rows = []
    with tempfile.TemporaryDirectory() as d:
        for src in _build.sources():
            out = _build.device_asm(src, os.path.join(d, os.path.basename(src) + ".s"))
            with open(out) as f:
                recs = asm_resources(f.read())
            for r, dem in zip(recs, _demangle([r["mangled"] for r in recs])):
                r["name"] = dem
                r["source"] = os.path.basename(src)
                rows.append(r)
    def norm(name):
        n = re.sub(r"^void\s+", "", name)
        n = n.replace("dg::(anonymous namespace)::", "").replace("dg::mfma::", "").replace("dg::q4::", "")
        return re.sub(r"\s+", "", n.split("(")[0])

    groups = collections.OrderedDict()
    for r in rows:
        r["norm"] = norm(r["name"])
        groups.setdefault((r["source"], re.sub(r"<.*", "", r["norm"])), []).append(r)

    def rng(rs, k):
        vals = [r.get(k, 0) for r in rs]
        lo, hi = min(vals), max(vals)
        return str(lo) if lo == hi else f"{lo}-{hi}"

    lines = ["# Compiler resource report of every kernel (gfx950)", "",
             "Command:", "", "    " + (command or "python -m memory_bound_decode_gemv_amd.profiling resources "
                                      "--md profiles/kernel_resources.md"), "",
             "From the \"; Kernel info\" block hipcc writes after each kernel in the device assembly "
             "(the same build flags as the library).  One line per kernel template: ranges over its "
             "instantiations.  `waves/SIMD` is the occupancy the registers allow (the compiler's "
             "\"Occupancy\"); LDS sized at launch (every staged kernel's buffers) is not part of it and "
             "lowers it further where a workgroup's LDS is large.  Scratch 0 everywhere means no spills.", "",
             f"{len(rows)} kernels in {len(groups)} templates.", "",
             "| source | kernel template | instantiations | VGPRs | AGPRs | SGPRs | static LDS B | scratch B | waves/SIMD |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (src, tmpl), rs in groups.items():
        lines.append(f"| {src} | `{tmpl}` | {len(rs)} | {rng(rs, 'vgpr')} | {rng(rs, 'agpr')} | {rng(rs, 'sgpr')} | "
                     f"{rng(rs, 'lds_static')} | {rng(rs, 'scratch')} | {rng(rs, 'occupancy')} |")
    lines += ["", "The instantiations the default dispatch launches for the headline and named workloads:", "",
              "| workload | kernel | VGPRs | SGPRs | waves/SIMD (registers) |", "|---|---|---|---|---|"]
    by_norm = {r["norm"]: r for r in rows}
    for label, key in DEFAULT_KERNELS:
        r = by_norm.get(key)
        if r is not None:
            lines.append(f"| {label} | `{key}` | {r.get('vgpr')} | {r.get('sgpr')} | {r.get('occupancy')} |")
    return "\n".join(lines) + "\n"


# (workload, kernel instantiation) of the default launches named in the report
DEFAULT_KERNELS = [
    ("fp16 GEMV 4096x4096", "k_gemv_wide<false,2,false,2>"),
    ("bf16 GEMV (decoder shapes, lm-head)", "k_gemv_wide<true,2,false,2>"),
    ("Q4_0 M=1 28672x8192", "k_q4_m1_ldsrow<2,5,2,false>"),
    ("Q4_0 M=16 4096x14336", "k_qmfma<FmtQ4_0,8,16,1,4,2>"),
    ("Q4_0 M=17..24 4096x14336", "k_qmfma<FmtQ4_0,8,24,1,12,1>"),
    ("Q4_0 M=9..16 14336x4096 (resident columns)", "k_qres<FmtQ4_0,1,4,2,2>"),
    ("NF4 M=1, K=8192", "k_nf4_rows<8,1>"),
    ("NF4 M=1, other K", "k_nf4_rows<4,1>"),
    ("Q8_1 quantiser", "k_quantize_q8_1"),
]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("fetch_csv")
    c.add_argument("write_csv")
    c.add_argument("--json", default=os.path.join(PROFILES, "counters.json"))
    c.add_argument("--md", default=os.path.join(PROFILES, "hbm_traffic_counters.md"))
    c.add_argument("--command-fetch", default="")
    c.add_argument("--command-write", default="")
    c.add_argument("--tcc", nargs="*", default=[], help="counter CSVs of the TCC request passes")
    c.add_argument("--command-tcc", default="")
    pm = sub.add_parser("pmc")
    pm.add_argument("csvs", nargs="+")
    pm.add_argument("--kernels", required=True)
    pm.add_argument("--labels", required=True)
    pm.add_argument("--per", type=int, default=4)
    pm.add_argument("--md", required=True)
    pm.add_argument("--command", default="")
    q = sub.add_parser("suite")
    q.add_argument("jsonl", nargs="+")
    q.add_argument("--md", required=True)
    q.add_argument("--command", default="")
    q.add_argument("--filter", default=None)
    q.add_argument("--condense", action="store_true",
                   help="one line per (workload, M): the default launch and the best configuration")
    lc = sub.add_parser("launchcost")
    lc.add_argument("trace_csv")
    lc.add_argument("--md", required=True)
    lc.add_argument("--command", default="")
    lc.add_argument("--labels", required=True, help="comma-separated workload names, in launch order")
    lc.add_argument("--bytes", required=True, help="comma-separated algorithmic bytes per launch, same order")
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("--md", required=True)
    t.add_argument("--command", default="")
    t.add_argument("--runs", default=None, help="kernel-trace CSV: add per-run durations")
    rs = sub.add_parser("resources")
    rs.add_argument("--md", default=os.path.join(PROFILES, "kernel_resources.md"))
    rs.add_argument("--command", default="")
    a = ap.parse_args(argv)
    if a.cmd == "resources":
        with open(a.md, "w") as f:
            f.write(resources_markdown(a.command))
        return 0
    if a.cmd == "counters":
        s = counters_summary(a.fetch_csv, a.write_csv, a.tcc)
        with open(a.json, "w") as f:
            json.dump(s, f, indent=1)
            f.write("\n")
        with open(a.md, "w") as f:
            f.write(counters_markdown(s, a.command_fetch, a.command_write, a.command_tcc))
        print(json.dumps(s, indent=1))
    elif a.cmd == "pmc":
        s = pmc_summary(a.csvs, a.kernels, a.labels.split(","), a.per)
        with open(a.md, "w") as f:
            f.write(pmc_markdown(s, a.command))
    elif a.cmd == "suite":
        with open(a.md, "w") as f:
            if a.condense:
                f.write(suite_condensed_markdown(a.jsonl, a.command, a.filter))
            else:
                f.write(suite_markdown(a.jsonl[0], a.command, a.filter))
    elif a.cmd == "launchcost":
        with open(a.md, "w") as f:
            f.write(launch_cost_markdown(a.trace_csv, a.command, a.labels.split(","),
                                         [int(x) for x in a.bytes.split(",")]))
    else:
        with open(a.md, "w") as f:
            f.write(trace_markdown(a.stats_csv, a.command, a.runs))
    return 0


if __name__ == "__main__":
    sys.exit(main())
