"""rocprofv3 driver and summariser for one Lloyd workload.

Runs ``bench.py`` under rocprofv3 three times, each pass a child process
under its own hard time limit, and writes short text summaries plus the
per-launch HBM traffic table that ``bench.py`` reports:

1. ``--kernel-trace --stats``: calls, average and minimum duration and
   share of GPU time per kernel, beside the per-phase times that bench.py
   measured with HIP events in the same run;
2. ``--pmc FETCH_SIZE``: KiB read from HBM per dispatch;
3. ``--pmc WRITE_SIZE``: KiB written to HBM per dispatch.

Each pass also runs bench.py's copy calibration: a plain elementwise kernel
(``dst = -src`` in fp32) over a buffer of known size, so that each counter's
reading converts to bytes by the ratio of the copy's known bytes to what the
counter reports for it.

Usage (on a machine with the GPU; the raw rocprofv3 output stays under
``--raw``)::

    python3 -m exact_means_clustering_flashassign_amd.profiling --workload api_example

This module only reads files and starts child processes; it never touches
the GPU itself.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import shlex
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
COPY_MIB = 1024
COPY_TAG = "neg_kernel"

# Kernel sources whose text decides a kernel's counter readings.
PHASE_SOURCES = {
    "assign": ("assign.hip", "assign_splitd.hip", "fk_internal.hpp"),
    "update": ("update.hip", "fk_internal.hpp"),
}


def source_digest(phase: str) -> str:
    h = hashlib.sha256()
    for name in PHASE_SOURCES[phase]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


BASELINE_KERNELS = ("argmin_rows_kernel", "scatter_add_kernel", "divide_kernel")


def phase_of(kernel: str) -> str:
    k = kernel.replace("(anonymous namespace)", "").split("(")[0]
    if (any(b in k for b in BASELINE_KERNELS) or k.startswith("Cijk_") or "rocblas" in k
            or ("zero_kernel" in k and "fk::" not in k)):
        return "baseline"
    if "assign_" in k:
        return "assign"
    if "norms_" in k and "_kernel" in k:
        return "norms"
    if COPY_TAG in k:
        return "copy"
    if "fk::" in k and ("widen_kernel" in k or "fill_i32_kernel" in k):
        return "setup"
    if "fk::" in k:
        return "update"
    return "other"


def short_name(kernel: str) -> str:
    k = (kernel.replace("fk::(anonymous namespace)::", "").replace("(anonymous namespace)::", "")
         .replace("void ", ""))
    head = k.split("(")[0]
    if COPY_TAG in k:
        return "torch neg_kernel (copy calibration)"
    if "at::native::" in k:
        return "torch " + k.split("at::native::")[-1].split("<")[0].split("(")[0][:60]
    return head[:70]


def _run(cmd, log, limit):
    """One profiled pass as a child process; returns its exit status."""
    env = dict(os.environ, TMPDIR="/tmp")
    full = ["timeout", "-s", "KILL", str(limit)] + cmd
    print("$ " + " ".join(shlex.quote(c) for c in full), flush=True)
    with open(log, "w") as f:
        r = subprocess.run(full, cwd="/tmp", env=env, stdout=f, stderr=subprocess.STDOUT)
    print(f"  rc={r.returncode}", flush=True)
    return r.returncode


def _bench_cmd(args):
    return ["python3", os.path.join(ROOT, "bench.py"), "--workload", args.workload,
            "--steps", str(args.steps), "--warmup", str(args.warmup), "--cpu-batches", "0",
            "--baselines", "0", "--tol-run", "0", "--copy-calibration", str(COPY_MIB)]


def _find(d, suffix):
    hits = glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def _bench_json(log):
    line = None
    with open(log) as f:
        for ln in f:
            if ln.startswith("{\"metric\""):
                line = ln
    return json.loads(line) if line else None


def read_stats(path):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"kernel": r["Name"], "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "total_ms": float(r["TotalDurationNs"]) / 1e6,
                         "pct": float(r["Percentage"])})
    return rows


def read_counter(path, counter):
    """Mean counter value per dispatch, by kernel name."""
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            s = acc.setdefault(r["Kernel_Name"], [0.0, 0])
            s[0] += float(r["Counter_Value"])
            s[1] += 1
    return {k: v[0] / v[1] for k, v in acc.items()}


def _cmd_lines(cmds):
    return ["  " + (c if isinstance(c, str) else " ".join(c)) for c in cmds]


def stats_text(cmds, rows, bench):
    out = ["rocprofv3 kernel statistics", "", "command (passes run from /tmp with TMPDIR=/tmp):"]
    out += _cmd_lines(cmds) + [""]
    if bench:
        cfg = bench["config"]["workload"]
        out += [f"workload: {cfg}", ""]
    out.append(f"{'kernel':72s} {'phase':7s} {'calls':>5s} {'avg us':>9s} {'min us':>9s} {'share':>6s}")
    for r in sorted(rows, key=lambda r: -r["total_ms"]):
        out.append(f"{short_name(r['kernel']):72s} {phase_of(r['kernel']):7s} {r['calls']:5d} "
                   f"{r['avg_us']:9.1f} {r['min_us']:9.1f} {r['pct']:5.1f}%")
    if bench and bench.get("gpu_baselines"):
        gb = bench["gpu_baselines"]
        out += ["", "same run, contrast baselines (each call on its own, same inputs, HIP events):"]
        out += [f"  {k}: {v:.4g}" if isinstance(v, float) else f"  {k}: {v}" for k, v in gb.items()]
    if bench:
        ph = bench["phases_ms"]
        out += ["", "same run, HIP events recorded by the library on the launch stream "
                    "(average per iteration over the timed region):"]
        out += [f"  {k:7s} {1e3 * v:9.1f} us" for k, v in ph.items()]
        out.append(f"  iter/s {bench['value']:.1f} (timed region under the tracer)")
    return "\n".join(out) + "\n"


def traffic_summary(fetch, write, nbytes_copy):
    """Per-kernel bytes per dispatch, scaled by the copy calibration."""
    cf = [v for k, v in fetch.items() if COPY_TAG in k]
    cw = [v for k, v in write.items() if COPY_TAG in k]
    if not cf or not cw:
        raise RuntimeError("copy-calibration kernel missing from the counter output")
    f_fetch = nbytes_copy / (cf[0] * 1024.0)
    f_write = nbytes_copy / (cw[0] * 1024.0)
    per = {}
    for k in set(fetch) | set(write):
        rd = fetch.get(k, 0.0) * 1024.0 * f_fetch
        wr = write.get(k, 0.0) * 1024.0 * f_write
        per[k] = {"fetch_kib": fetch.get(k, 0.0), "write_kib": write.get(k, 0.0),
                  "read_bytes": rd, "write_bytes": wr, "phase": phase_of(k)}
    return per, f_fetch, f_write


def traffic_text(cmds, per, f_fetch, f_write, nbytes_copy, algo):
    out = ["rocprofv3 HBM traffic per dispatch (FETCH_SIZE, WRITE_SIZE)", "",
           "command (passes run from /tmp with TMPDIR=/tmp):"]
    out += _cmd_lines(cmds)
    out += ["", f"calibration: dst = -src over {nbytes_copy / 2**20:.0f} MiB fp32 reads and writes "
                f"{nbytes_copy:.0f} B each way;",
            f"  bytes per counter KiB: FETCH_SIZE x{f_fetch:.3f}, WRITE_SIZE x{f_write:.3f}", ""]
    out.append(f"{'kernel':72s} {'phase':7s} {'FETCH KiB':>11s} {'WRITE KiB':>11s} {'read MB':>9s} {'write MB':>9s}")
    for k, v in sorted(per.items(), key=lambda kv: -(kv[1]["read_bytes"] + kv[1]["write_bytes"])):
        out.append(f"{short_name(k):72s} {v['phase']:7s} {v['fetch_kib']:11.0f} {v['write_kib']:11.0f} "
                   f"{v['read_bytes'] / 1e6:9.2f} {v['write_bytes'] / 1e6:9.2f}")
    out.append("")
    for ph, a in algo.items():
        meas = sum(v["read_bytes"] + v["write_bytes"] for v in per.values() if v["phase"] == ph)
        out.append(f"{ph}: measured {meas / 1e6:.1f} MB per launch vs algorithmic {a / 1e6:.1f} MB "
                   f"(x{meas / a:.2f})")
    return "\n".join(out) + "\n"


def baselines_pass(args) -> int:
    """Kernel statistics of a short bench run with the contrast baselines."""
    wl = args.workload
    raw = os.path.join(args.raw, wl)
    os.makedirs(raw, exist_ok=True)
    os.makedirs(args.out, exist_ok=True)
    bcmd = ["python3", os.path.join(ROOT, "bench.py"), "--workload", wl, "--steps", "2",
            "--warmup", "1", "--cpu-batches", "0", "--tol-run", "0", "--baselines", "1"]
    cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
           os.path.join(raw, "baselines"), "-o", "run", "--"] + bcmd
    log = os.path.join(raw, "baselines.log")
    if not args.summarize_only:
        rc = _run(cmd, log, args.limit)
        if rc != 0:
            return rc
    top = _top_line(args, "--baselines --workload " + wl)
    rows = read_stats(_find(os.path.join(raw, "baselines"), "_kernel_stats.csv"))
    txt = stats_text([top, "  which runs:", cmd], rows, _bench_json(log))
    txt = txt.replace(ROOT + "/", "")
    with open(os.path.join(args.out, f"kernels_baselines_{wl}.txt"), "w") as f:
        f.write(txt)
    print(txt, flush=True)
    return 0


# Counters of the MFMA-utilisation pass: the MFMA pipe's busy cycles, the
# GPU's busy clock cycles, and what the LDS and the VALU issue. One pass holds
# at most 8 SQ and 2 GRBM counters.
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU",
                 "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT",
                 "GRBM_GUI_ACTIVE")
PROBE_TAG = "mfma_peak_kernel"
SIMDS_PER_CU = 4
# Second pass: where the waves' cycles go (issue, waits by kind, MFMA
# co-execution with other VALU work).
STALL_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                  "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM",
                  "SQ_VALU_MFMA_COEXEC_CYCLES", "GRBM_GUI_ACTIVE")
# Third pass (the workload only): how busy the LDS is. SQ_LDS_IDX_ACTIVE
# counts the cycles each CU's LDS serves indexed reads and writes.
LDS_COUNTERS = ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL",
                "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_INSTS_LDS_STORE_BANDWIDTH",
                "SQ_LDS_ADDR_CONFLICT", "SQ_LDS_UNALIGNED_STALL", "GRBM_GUI_ACTIVE")


def read_dispatch_counters(path):
    """Counter values per dispatch: {dispatch id: {"kernel": name, counter: value}}."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            e = out.setdefault(r["Dispatch_Id"], {"kernel": r["Kernel_Name"]})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def read_dispatch_durations(path):
    """Kernel durations in ns per dispatch id, from a kernel-trace csv."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            out[r["Dispatch_Id"]] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return out


def counter_means(disp, durs, select):
    """Mean counter values and duration over the dispatches whose kernel name
    satisfies `select`; None if there are none."""
    rows = [dict(e, dur_ns=durs.get(i)) for i, e in disp.items() if select(e["kernel"])]
    if not rows:
        return None
    keys = [k for k in rows[0] if k != "kernel"]
    m = {k: sum(r[k] for r in rows if r.get(k) is not None) /
         max(1, sum(1 for r in rows if r.get(k) is not None)) for k in keys}
    m["kernel"] = rows[0]["kernel"]
    m["dispatches"] = len(rows)
    return m


def mfma_derived(m, cus, flop_per_launch=None, peak_tflops=None, nominal_mhz=2400.0,
                 xcds=8):
    """Clock and MFMA utilisation from one kernel's mean counters.
    GRBM_GUI_ACTIVE is summed over the XCDs (each has its own GRBM), so one
    XCD's busy cycles are GRBM_GUI_ACTIVE / xcds.
      clock (MHz)     = GRBM_GUI_ACTIVE / xcds / kernel duration (us)
      MFMA busy       = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / xcds * CUs * 4 SIMDs)
      achieved        = flop per launch / duration
      frac at clock   = achieved / (peak * clock / nominal clock)
      LDS busy        = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / xcds * CUs)"""
    d = {}
    g = m.get("GRBM_GUI_ACTIVE")
    dur = m.get("dur_ns")
    cyc = g / xcds if g else None
    if cyc and dur:
        d["clock_mhz"] = cyc / (dur / 1e3)
    if cyc and m.get("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
        d["mfma_busy"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * cus * SIMDS_PER_CU)
    if cyc and m.get("SQ_VALU_MFMA_COEXEC_CYCLES") is not None:
        d["mfma_coexec"] = m["SQ_VALU_MFMA_COEXEC_CYCLES"] / (cyc * cus * SIMDS_PER_CU)
    if cyc and m.get("SQ_LDS_IDX_ACTIVE") is not None:
        d["lds_util"] = m["SQ_LDS_IDX_ACTIVE"] / (cyc * cus)
        if m.get("SQ_INSTS_LDS_LOAD_BANDWIDTH") is not None:
            # 64-byte units read per CU per busy cycle
            d["lds_read_bytes_per_cu_cycle"] = 64 * m["SQ_INSTS_LDS_LOAD_BANDWIDTH"] / (cyc * cus)
    w = m.get("SQ_WAVE_CYCLES")
    if w:
        for k in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_WAIT_INST_LDS"):
            if m.get(k) is not None:
                d[k.replace("SQ_", "").lower() + "_per_wave_cycle"] = m[k] / w
    if flop_per_launch and dur:
        d["achieved_tflops"] = flop_per_launch / (dur * 1e-9) / 1e12
        if peak_tflops:
            d["frac_of_nominal"] = d["achieved_tflops"] / peak_tflops
            if "clock_mhz" in d:
                d["frac_at_clock"] = d["achieved_tflops"] / (peak_tflops * d["clock_mhz"] /
                                                             nominal_mhz)
    return d


def counters_text(cmds, entries, cus, xcds=8):
    out = ["rocprofv3 counters: MFMA utilisation and clock", "",
           "command (passes run from /tmp with TMPDIR=/tmp):"]
    out += _cmd_lines(cmds)
    out += ["", f"compute units: {cus} in {xcds} XCDs; GRBM_GUI_ACTIVE is summed over the XCDs;",
            f"clock = GRBM_GUI_ACTIVE / {xcds} / kernel duration;",
            f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {xcds} x {cus} CUs x "
            f"{SIMDS_PER_CU} SIMDs);",
            "frac at clock = achieved / (nominal peak x measured clock / 2400 MHz);",
            "*_per_wave_cycle = counter / SQ_WAVE_CYCLES (second pass);",
            f"LDS busy = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / {xcds} x {cus} CUs) (third pass).",
            ""]
    for name, e in entries.items():
        m, dv = e["means"], e["derived"]
        out.append(f"{name}: {short_name(m['kernel'])} ({m['dispatches']} dispatches"
                   + (f", kernel source digest {e['digest']}" if e.get("digest") else "") + ")")
        out.append(f"  duration avg {m.get('dur_ns', 0) / 1e3:.1f} us")
        for k in dict.fromkeys(MFMA_COUNTERS + STALL_COUNTERS + LDS_COUNTERS):
            if k in m:
                out.append(f"  {k:28s} {m[k]:.6g}")
        for k, v in dv.items():
            out.append(f"  {k:28s} {v:.4g}")
        out.append("")
    return "\n".join(out) + "\n"


def counters_pass(args) -> int:
    """MFMA utilisation and stall attribution of the assign kernel of a
    workload, next to the same counters for the MFMA peak probe (bench.py
    --mfma-peak). Each counter set runs in its own rocprofv3 process with
    --pmc and --kernel-trace (durations per dispatch)."""
    sys.path.insert(0, ROOT)
    import bench

    wl = args.workload
    raw = os.path.join(args.raw, wl)
    os.makedirs(raw, exist_ok=True)
    os.makedirs(args.out, exist_ok=True)
    wcmd = ["python3", os.path.join(ROOT, "bench.py"), "--workload", wl, "--steps",
            str(args.steps), "--warmup", str(args.warmup), "--cpu-batches", "0", "--baselines", "0",
            "--tol-run", "0"]
    pcmd = ["python3", os.path.join(ROOT, "bench.py"), "--mfma-peak", "--steps", "3",
            "--peak-iters", "4000"]
    sets = {"mfma": args.counter_list.split(","), "stalls": list(STALL_COUNTERS),
            "lds": list(LDS_COUNTERS)}
    passes = {}
    for prog, cmd in (("workload", wcmd), ("probe", pcmd)):
        for cset, ctrs in sets.items():
            if prog == "probe" and cset == "lds":
                continue                   # the probe touches no LDS
            tag = f"counters_{cset}_{prog}"
            passes[tag] = (["rocprofv3", "--pmc", *ctrs, "--kernel-trace", "--output-format",
                            "csv", "-d", os.path.join(raw, tag), "-o", "run", "--"] + cmd)
    if not args.summarize_only:
        with open(os.path.join(raw, "counters_sources.json"), "w") as f:
            json.dump({ph: source_digest(ph) for ph in PHASE_SOURCES}, f)
        for tag, cmd in passes.items():
            rc = _run(cmd, os.path.join(raw, tag + ".log"), min(args.limit, 180))
            if rc != 0:
                return rc
    with open(os.path.join(raw, "counters_sources.json")) as f:
        digests = json.load(f)
    from synthdata import SHAPES
    B, N, d_, K, dt, _, _ = SHAPES[wl]
    flop = bench.assign_flop(B, N, d_, K)
    peak = bench.PEAK_MFMA_F32 if dt == "f32" else bench.PEAK_MFMA_F16
    merged = {"workload": {}, "probe": {}}
    probe_flop = None
    for tag in passes:
        prog = tag.rsplit("_", 1)[1]
        disp = read_dispatch_counters(_find(os.path.join(raw, tag), "_counter_collection.csv"))
        durs = read_dispatch_durations(_find(os.path.join(raw, tag), "_kernel_trace.csv"))
        if prog == "workload":
            m = counter_means(disp, durs, lambda k: phase_of(k) == "assign")
        else:
            m = counter_means(disp, durs, lambda k: PROBE_TAG in k)
            pj = _bench_json(os.path.join(raw, tag + ".log")) or {}
            cfg = pj.get("config", {})
            # blocks x 4 waves x iters x 32 MFMAs of 32768 flop (the probe's grid)
            probe_flop = (cfg.get("blocks", 0) * 4.0 * cfg.get("iters", 0) * 32 * 32768) or None
        if m:
            e = merged[prog]
            dur = e.get("dur_ns")
            e.update(m)
            if dur is not None:        # the first pass's duration (the MFMA counter set)
                e["dur_ns"] = dur
    entries = {}
    if merged["workload"]:
        m = merged["workload"]
        entries[f"assign ({wl})"] = {"means": m, "digest": digests["assign"],
                                     "derived": mfma_derived(m, args.cus, flop, peak)}
    if merged["probe"]:
        m = merged["probe"]
        entries["mfma peak probe"] = {"means": m, "derived": mfma_derived(
            m, args.cus, probe_flop, bench.PEAK_MFMA_F16)}
    top = _top_line(args, "--counters --workload " + wl)
    txt = counters_text([top, "  which runs:"] + list(passes.values()),
                        entries, args.cus).replace(ROOT + "/", "")
    with open(os.path.join(args.out, f"counters_{wl}.txt"), "w") as f:
        f.write(txt)
    print(txt, flush=True)
    cpath = os.path.join(args.out, "counters.json")
    table = {}
    for base in (os.path.join(ROOT, "profiles", "counters.json"), cpath):
        try:
            with open(base) as f:
                table.update(json.load(f))
        except (OSError, ValueError):
            pass
    table[wl] = {k: {"kernel_source_digest": v.get("digest"), **v["derived"],
                     "duration_us": v["means"].get("dur_ns", 0) / 1e3}
                 for k, v in entries.items()}
    with open(cpath, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    return 0


def _top_line(args, what):
    """The command line that reproduces these passes, with the output folders
    given relative to the repository root."""
    rel = [os.path.relpath(os.path.abspath(p), ROOT) for p in (args.out, args.raw)]
    return ("python3 -m exact_means_clustering_flashassign_amd.profiling " + what
            + f" --out {rel[0]} --raw {rel[1]}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="api_example")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--out", default=os.path.join(ROOT, "prof_out", "profiles"),
                    help="where the text summaries and traffic.json go")
    ap.add_argument("--raw", default=os.path.join(ROOT, "prof_out", "rocprof"),
                    help="where rocprofv3 writes its raw output")
    ap.add_argument("--limit", type=int, default=240, help="seconds per pass")
    ap.add_argument("--summarize-only", action="store_true",
                    help="do not run anything; summarise the raw output of an earlier run")
    ap.add_argument("--baselines", action="store_true",
                    help="instead: one kernel-statistics pass of a short run that also times "
                         "the contrast baselines (kernels_baselines_<workload>.txt)")
    ap.add_argument("--counters", action="store_true",
                    help="instead: the MFMA-utilisation counter pass of the workload's assign and "
                         "of the MFMA peak probe (counters_<workload>.txt)")
    ap.add_argument("--counter-list", default=",".join(MFMA_COUNTERS),
                    help="counters of the --counters pass (at most 8 SQ_ and 2 GRBM_)")
    ap.add_argument("--cus", type=int, default=256, help="compute units of the GPU")
    args = ap.parse_args(argv)
    # the passes run from /tmp: output folders are fixed against the caller's cwd
    args.out, args.raw = os.path.abspath(args.out), os.path.abspath(args.raw)
    if args.baselines:
        return baselines_pass(args)
    if args.counters:
        return counters_pass(args)
    sys.path.insert(0, ROOT)
    import bench  # algorithmic byte counts; bench imports torch lazily

    wl = args.workload
    raw = os.path.join(args.raw, wl)
    os.makedirs(raw, exist_ok=True)
    os.makedirs(args.out, exist_ok=True)
    bcmd = _bench_cmd(args)
    top = _top_line(args, "--workload " + wl)
    passes = {
        "stats": ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                  os.path.join(raw, "stats"), "-o", "run", "--"] + bcmd,
        "fetch_size": ["rocprofv3", "--pmc", "FETCH_SIZE", "--output-format", "csv", "-d",
                       os.path.join(raw, "fetch_size"), "-o", "run", "--"] + bcmd,
        "write_size": ["rocprofv3", "--pmc", "WRITE_SIZE", "--output-format", "csv", "-d",
                       os.path.join(raw, "write_size"), "-o", "run", "--"] + bcmd,
    }
    meta_path = os.path.join(raw, "sources.json")
    if not args.summarize_only:
        with open(meta_path, "w") as f:
            json.dump({ph: source_digest(ph) for ph in PHASE_SOURCES}, f)
        for name, cmd in passes.items():
            rc = _run(cmd, os.path.join(raw, name + ".log"), args.limit if name == "stats" else min(args.limit, 120))
            if rc != 0:
                return rc
    with open(meta_path) as f:
        digests = json.load(f)

    def clean(t):
        return t.replace(ROOT + "/", "")

    rows = read_stats(_find(os.path.join(raw, "stats"), "_kernel_stats.csv"))
    txt = stats_text([top, "  which runs:", passes["stats"]], rows,
                     _bench_json(os.path.join(raw, "stats.log")))
    with open(os.path.join(args.out, f"kernels_{wl}.txt"), "w") as f:
        f.write(clean(txt))
    print(clean(txt), flush=True)

    counters = {ctr: read_counter(_find(os.path.join(raw, ctr.lower()), "_counter_collection.csv"), ctr)
                for ctr in ("FETCH_SIZE", "WRITE_SIZE")}
    nbytes = COPY_MIB * 2**20
    per, ff, fw = traffic_summary(counters["FETCH_SIZE"], counters["WRITE_SIZE"], nbytes)
    from synthdata import SHAPES
    B, N, d_, K, dt, _, _ = SHAPES[wl]
    s = bench.elem_bytes(dt)
    algo = {"assign": bench.assign_bytes(B, N, d_, K, s), "update": bench.update_bytes(B, N, d_, K, s)}
    txt = traffic_text([top, "  which runs:", passes["fetch_size"], passes["write_size"]], per, ff, fw,
                       nbytes, algo)
    with open(os.path.join(args.out, f"traffic_{wl}.txt"), "w") as f:
        f.write(clean(txt))
    print(clean(txt), flush=True)

    tpath = os.path.join(args.out, "traffic.json")
    table = {}
    for base in (os.path.join(ROOT, "profiles", "traffic.json"), tpath):   # keep other workloads
        try:
            with open(base) as f:
                table.update(json.load(f))
        except (OSError, ValueError):
            pass
    entry = {"factor_fetch": ff, "factor_write": fw}
    for ph in ("assign", "update"):
        rd = sum(v["read_bytes"] for v in per.values() if v["phase"] == ph)
        wr = sum(v["write_bytes"] for v in per.values() if v["phase"] == ph)
        entry[ph] = {"kernel_source_digest": digests[ph], "read_bytes": rd, "write_bytes": wr,
                     "hbm_bytes_per_launch": rd + wr}
    table[wl] = entry
    with open(tpath, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
