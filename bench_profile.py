#!/usr/bin/env python3
"""Summarise rocprofv3 results of bench.py into profiles/.

    python bench_profile.py --name qwen3_8b_q32 --cmd-trace "..." --trace DIR \
        [--fetch DIR --write DIR --cmd-pmc "..."]

DIR is a rocprofv3 output directory (-d) holding a *_results.db written by
--kernel-trace (and --pmc).  Writes:
  profiles/<name>_kernel_trace.md   per-kernel calls and durations
  profiles/<name>_hbm_traffic.md    FETCH_SIZE / WRITE_SIZE per launch, the
                                    calibration against a 1 GiB device copy,
                                    and calibrated HBM bytes per launch
  profiles/traffic.json             the calibrated bytes per launch of the
                                    projection kernel, tagged with the kernel
                                    source hash (bench.py reports them only
                                    while that hash matches)
Runs on the host only; it reads the databases, it launches nothing.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sqlite3
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(HERE, "profiles")
COPY_BYTES = 1 << 30   # bench.py --calibration-copy copies 2^28 int32


def kernel_source_hash():
    """Hash of the kernels' sources (aa_kernels.hip, aa_small.hip,
    aa_backward.hip, aa_tile32.hip and the device header they include): stored
    traffic figures are used only while it matches."""
    h = hashlib.sha256()
    for name in ("aa_kernels.hip", "aa_small.hip", "aa_backward.hip", "aa_tile32.hip", "aa_device.h"):
        with open(os.path.join(HERE, "associative_algebra_block_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _db(d):
    dbs = sorted(glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no *_results.db under {d}")
    return sqlite3.connect(dbs[-1])


def short(name, n=96):
    return name if len(name) <= n else name[:n - 3] + "..."


def kernel_stats(d):
    c = _db(d)
    rows = c.execute("select name, grid_x, workgroup_x, count(*), avg(end - start), min(end - start), "
                     "max(end - start), sum(end - start) from kernels group by name, grid_x "
                     "order by sum(end - start) desc").fetchall()
    total = sum(r[7] for r in rows) or 1
    return [dict(name=r[0], grid=r[1], wg=r[2], calls=r[3], avg_us=r[4] / 1e3, min_us=r[5] / 1e3,
                 max_us=r[6] / 1e3, total_us=r[7] / 1e3, pct=100.0 * r[7] / total) for r in rows]


def pmc(d, counter):
    """Mean counter value per kernel name, and the largest single dispatch."""
    c = _db(d)
    out = {}
    for name, val in c.execute("select name, counter_value from pmc_events where counter_name = ?", (counter,)):
        out.setdefault(name, []).append(val)
    return {k: statistics.mean(v) for k, v in out.items()}, {k: max(v) for k, v in out.items()}




def bench_record(log):
    rec = None
    with open(log) as f:
        for line in f:
            if line.startswith('{"metric"'):
                rec = json.loads(line)
    if rec is None:
        raise SystemExit(f"no bench.py result line in {log}")
    return rec


def last_calls(d, match, n):
    """Name, count and mean duration (us) of the last n dispatches of the
    longest-running kernel whose name contains `match`."""
    c = _db(d)
    names = [r[0] for r in c.execute("select name, sum(end - start) s from kernels group by name order by s desc")
             if match in r[0]]
    if not names:
        return None
    durs = [r[0] for r in c.execute("select end - start from kernels where name = ? order by start", (names[0],))]
    tail = durs[-n:]
    return names[0], len(tail), sum(tail) / len(tail) / 1e3


def bench_durations(log):
    """Per-call durations (ms) from the JSON line bench.py printed."""
    rec = bench_record(log)
    if "parts" in rec:
        return {k: v["ms"] for k, v in rec["parts"].items()}
    if "kernel_ms" not in rec:
        return {}
    return {"swiglu_ffn" if "SwiGLU" in rec.get("metric", "") else "projection": rec["kernel_ms"]}


def is_calibration_copy(name):
    return "copyBuffer" in name or "copy_kernel" in name or "CopyKernel" in name


def write_counters(a, src):
    """Per-kernel means of the counters of one --pmc run, with the kernel's
    mean duration and GRBM_GUI_ACTIVE-normalised busy fractions where the
    counters allow (SQ counters read one of the 32 shader engines: 8 CUs, 32
    SIMDs; SQ_*_CYCLES wave and busy counters count in units of 4 cycles)."""
    c = _db(a.counters)
    rows = c.execute("select name, counter_name, avg(counter_value), avg(duration) from pmc_events "
                     "group by name, counter_name").fetchall()
    per = {}
    for name, cn, v, dur in rows:
        if a.match and a.match not in name:
            continue
        d = per.setdefault(name, {"_us": dur / 1000.0})
        d[cn] = v
    names = sorted({cn for d in per.values() for cn in d if not cn.startswith("_")})
    lines = [f"# Counters: {a.name}", "", f"Command (run from /tmp with TMPDIR=/tmp): `{a.cmd_counters}`", "",
             f"Kernel sources (aa_kernels.hip, aa_small.hip, aa_backward.hip, aa_tile32.hip, aa_device.h) sha256[:16]: `{src}`", "",
             "Mean per dispatch.  SQ counters read one of the 32 shader engines (8 CUs, 32 SIMDs).  "
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (32 x GRBM_GUI_ACTIVE); wait share = SQ_WAIT_INST_ANY / "
             "SQ_WAVE_CYCLES (waves waiting on their own loads); residency = 4 x SQ_WAVE_CYCLES / "
             "(SIMDs x waves per SIMD x GRBM_GUI_ACTIVE) is not shown, the occupancy differs per kernel.", "",
             "| kernel | us | " + " | ".join(names) + " | MFMA busy | wait share |",
             "|---|---|" + "---|" * len(names) + "---|---|"]
    for n, d in sorted(per.items(), key=lambda kv: -kv[1]["_us"]):
        mf = d.get("SQ_VALU_MFMA_BUSY_CYCLES"), d.get("GRBM_GUI_ACTIVE")
        busy = f"{mf[0] / (32 * mf[1]):.3f}" if mf[0] is not None and mf[1] else "-"
        wt = d.get("SQ_WAIT_INST_ANY"), d.get("SQ_WAVE_CYCLES")
        wait = f"{wt[0] / wt[1]:.3f}" if wt[0] is not None and wt[1] else "-"
        lines.append(f"| `{short(n)}` | {d['_us']:.2f} | " + " | ".join(f"{d.get(k, 0):.0f}" for k in names) +
                     f" | {busy} | {wait} |")
    with open(os.path.join(PROFILES, f"{a.name}_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--name", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--cmd-trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--cmd-pmc", default="")
    ap.add_argument("--key", default=None, help="traffic.json key for the projection kernel")
    ap.add_argument("--alg-bytes", type=float, default=None, help="algorithmic bytes per projection launch")
    ap.add_argument("--match", default="leaf_", help="substring naming the projection kernel instance")
    ap.add_argument("--bench-log", default=None,
                    help="output of the same bench.py command run without the tracer just before")
    ap.add_argument("--bench-log-traced", default=None, help="output of the traced bench.py run")
    ap.add_argument("--counters", default=None,
                    help="a rocprofv3 --pmc output directory: write profiles/<name>_counters.md, the mean of every "
                         "counter per kernel (only kernels whose name contains --match)")
    ap.add_argument("--cmd-counters", default="")
    a = ap.parse_args()
    os.makedirs(PROFILES, exist_ok=True)
    src = kernel_source_hash()
    if a.counters:
        write_counters(a, src)

    ks = kernel_stats(a.trace)
    lines = [f"# Kernel trace: {a.name}", "",
             f"Command (run from /tmp with TMPDIR=/tmp): `{a.cmd_trace}`", "",
             f"Kernel sources (aa_kernels.hip, aa_small.hip, aa_backward.hip, aa_tile32.hip, aa_device.h) sha256[:16]: `{src}`", "",
             "| kernel | grid (threads) | calls | avg us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|---|"]
    for k in ks:
        lines.append(f"| `{short(k['name'])}` | {k['grid']} | {k['calls']} | {k['avg_us']:.2f} | "
                     f"{k['min_us']:.2f} | {k['max_us']:.2f} | {k['pct']:.1f} |")
    if a.bench_log or a.bench_log_traced:
        plain = bench_durations(a.bench_log) if a.bench_log else {}
        traced = bench_durations(a.bench_log_traced) if a.bench_log_traced else {}
        lines += ["", "bench.py's own durations of each call, mean over its timed calls (HIP events: the start "
                      "event is a marker recorded just before the call's first dispatch, the stop event is "
                      "recorded by its last kernel).  Under the tracer every dispatch starts 4-5 us after the "
                      "marker before it, a gap the trace's kernel durations do not contain; without the tracer "
                      "the same command gives the first column.  The trace's averages above also hold the "
                      "warmup calls.", "",
                      "| call | bench.py, no tracer (same command, run just before) | bench.py in the traced run |",
                      "|---|---|---|"]
        for k in sorted(set(plain) | set(traced), key=lambda k: list(plain or traced).index(k)):
            f = lambda d: f"{d[k] * 1e3:.2f} us" if k in d else "-"
            lines.append(f"| {k} | {f(plain)} | {f(traced)} |")
        if a.bench_log_traced and a.match:
            lc = last_calls(a.trace, a.match, int(bench_record(a.bench_log_traced)["steps"]))
            if lc:
                lines += ["", f"Trace average of `{short(lc[0], 60)}` over its last {lc[1]} dispatches (the "
                              f"timed steps, one call each): {lc[2]:.2f} us."]
    with open(os.path.join(PROFILES, f"{a.name}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:14]))

    if a.fetch and a.write:
        (fe, fe_max), (wr, wr_max) = pmc(a.fetch, "FETCH_SIZE"), pmc(a.write, "WRITE_SIZE")
        cal = [n for n in fe if is_calibration_copy(n)]
        if not cal:
            raise SystemExit("no calibration copy kernel in the FETCH_SIZE run (use bench.py --calibration-copy)")
        # the 1 GiB copies are the largest dispatches of the copy kernel
        # (smaller copies in the same run share its name)
        cname = max(cal, key=lambda n: wr_max.get(n, 0))
        f_fac = COPY_BYTES / (fe_max[cname] * 1024.0)
        w_fac = COPY_BYTES / (wr_max[cname] * 1024.0)
        fe[cname], wr[cname] = fe_max[cname], wr_max[cname]
        lines = [f"# HBM traffic per launch: {a.name}", "",
                 f"Commands (run from /tmp with TMPDIR=/tmp): `{a.cmd_pmc.replace('PMC', 'FETCH_SIZE')}` and "
                 f"`{a.cmd_pmc.replace('PMC', 'WRITE_SIZE')}`", "",
                 f"Kernel sources (aa_kernels.hip, aa_small.hip, aa_backward.hip, aa_tile32.hip, aa_device.h) sha256[:16]: `{src}`", "",
                 f"Calibration: a 1 GiB device copy (`{short(cname, 60)}`, its largest dispatches) reads FETCH_SIZE = {fe[cname]:.0f} KiB "
                 f"and WRITE_SIZE = {wr[cname]:.0f} KiB per launch, so bytes = FETCH_SIZE x 1024 x {f_fac:.4f} "
                 f"and WRITE_SIZE x 1024 x {w_fac:.4f}.", "",
                 "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | write MB | total MB |",
                 "|---|---|---|---|---|---|"]
        traffic = {}
        for n in sorted(set(fe) | set(wr), key=lambda n: -(fe.get(n, 0) + wr.get(n, 0))):
            r = fe.get(n, 0) * 1024 * f_fac
            w = wr.get(n, 0) * 1024 * w_fac
            lines.append(f"| `{short(n)}` | {fe.get(n, 0):.0f} | {wr.get(n, 0):.0f} | {r / 1e6:.2f} | "
                         f"{w / 1e6:.2f} | {(r + w) / 1e6:.2f} |")
            if a.match in n and not traffic:   # the largest matching kernel
                traffic = {"read_bytes": r, "write_bytes": w, "hbm_bytes_per_launch": r + w, "kernel": n}
        if traffic and a.alg_bytes:
            lines += ["", f"`{short(traffic['kernel'], 60)}`: {traffic['hbm_bytes_per_launch'] / 1e6:.2f} MB measured per launch "
                          f"against {a.alg_bytes / 1e6:.2f} MB algorithmic "
                          f"({traffic['hbm_bytes_per_launch'] / a.alg_bytes:.3f}x)."]
        with open(os.path.join(PROFILES, f"{a.name}_hbm_traffic.md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))
        if traffic and a.key:
            p = os.path.join(PROFILES, "traffic.json")
            rec = {}
            if os.path.exists(p):
                with open(p) as f:
                    rec = json.load(f)
            if rec.get("kernel_source_sha256_16") != src:
                rec = {"kernel_source_sha256_16": src, "kernels": {}}
            rec["kernels"][a.key] = {k: (round(v) if isinstance(v, float) else v) for k, v in traffic.items()}
            rec["calibration"] = {"fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
                                  "reference": "1 GiB device-to-device copy in the same run"}
            with open(p, "w") as f:
                json.dump(rec, f, indent=1)


if __name__ == "__main__":
    main()
