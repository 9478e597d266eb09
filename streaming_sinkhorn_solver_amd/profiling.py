"""Summaries of rocprofv3 databases (rocpd SQLite) for the solver's kernels.

    python -m streaming_sinkhorn_solver_amd.profiling stats DB OUT.md --command "..."
    python -m streaming_sinkhorn_solver_amd.profiling traffic FETCH_DB WRITE_DB OUT.json \
        --copy-bytes B --kernel lse_mfma_kernel --source fs_lse.hip \
        --command-fetch "..." --command-write "..."
    python -m streaming_sinkhorn_solver_amd.profiling counters OUT.md --db P1 --db P2 \
        --kernel lse_mfma_kernel --command "..." --command "..."

`stats` tabulates kernel-trace durations (calls, mean, min, max, share).
`counters` tabulates the mean per dispatch of every counter of one kernel over
several counter passes, with the clock and matrix-pipe share derived from them.
`traffic` turns the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) of one
kernel into HBM bytes per launch, each scaled by the factor that makes the
same counter read exactly the known size of a plain copy in the same run
(a 1 GiB elementwise read + write issued by the benchmark's counter mode).
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import sqlite3
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def kernel_source_sha(name: str = "fs_lse.hip") -> str:
    """First 16 hex digits of the SHA-256 of a kernel source under csrc/."""
    with open(os.path.join(HERE, "csrc", name), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def kernel_stats(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels").fetchall()
    agg = collections.OrderedDict()
    for name, dur in rows:
        a = agg.setdefault(name, [0, 0.0, float("inf"), 0.0])
        a[0] += 1
        a[1] += dur
        a[2] = min(a[2], dur)
        a[3] = max(a[3], dur)
    total = sum(v[1] for v in agg.values()) or 1.0
    out = [(n, c, t, t / c, mn, mx, t / total) for n, (c, t, mn, mx) in agg.items()]
    out.sort(key=lambda r: -r[2])
    return out


def write_stats_md(db: str, out_md: str, command: str) -> None:
    st = kernel_stats(db)
    lines = [f"# Kernel trace summary: {os.path.basename(out_md)}", "",
             "Command (run from the repository root on one MI355X):", "",
             "```", command, "```", "",
             "| kernel | calls | total ms | mean us | min us | max us | share |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for n, c, t, avg, mn, mx, share in st:
        lines.append(f"| `{n[:110]}` | {c} | {t / 1e6:.3f} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | "
                     f"{mx / 1e3:.1f} | {100 * share:.2f}% |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def counter_per_dispatch(db: str, counter: str, name_substr: str):
    """Mean over matching dispatches of the counter summed over its instances,
    plus the number of dispatches."""
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, dispatch_id, counter_name, value "
                       "from counters_collection").fetchall()
    per = collections.defaultdict(float)
    for kn, did, cn, v in rows:
        if cn == counter and name_substr in kn:
            per[did] += v
    if not per:
        raise KeyError(f"no {counter} values for kernels matching {name_substr!r} in {db}")
    return sum(per.values()) / len(per), len(per)


def write_traffic(fetch_db: str, write_db: str, out_json: str, copy_bytes: float,
                  kernel: str, copy_kernel: str, commands: dict,
                  source: str = "fs_lse.hip") -> dict:
    kib = 1024.0
    f_k, nf = counter_per_dispatch(fetch_db, "FETCH_SIZE", kernel)
    w_k, nw = counter_per_dispatch(write_db, "WRITE_SIZE", kernel)
    f_c, _ = counter_per_dispatch(fetch_db, "FETCH_SIZE", copy_kernel)
    w_c, _ = counter_per_dispatch(write_db, "WRITE_SIZE", copy_kernel)
    ff = copy_bytes / (f_c * kib)
    fw = copy_bytes / (w_c * kib)
    rec = {
        "kernel": kernel, "kernel_source": source, "kernel_source_sha": kernel_source_sha(source),
        "fetch_kib_per_launch_raw": f_k, "write_kib_per_launch_raw": w_k,
        "copy_bytes": copy_bytes, "copy_fetch_kib_raw": f_c, "copy_write_kib_raw": w_c,
        "fetch_scale": ff, "write_scale": fw,
        "hbm_fetch_bytes_per_launch": f_k * kib * ff,
        "hbm_write_bytes_per_launch": w_k * kib * fw,
        "hbm_bytes_per_launch": f_k * kib * ff + w_k * kib * fw,
        "launches": [nf, nw], "commands": commands,
    }
    with open(out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def kernel_durations(db: str, name_substr: str):
    """Durations (ns) of the dispatches of matching kernels, by dispatch id
    (empty if the database holds no kernel trace)."""
    con = sqlite3.connect(db)
    try:
        rows = con.execute("select name, dispatch_id, duration from kernels").fetchall()
    except sqlite3.Error:
        return {}
    return {did: dur for name, did, dur in rows if name_substr in name}


def write_counters_md(dbs, out_md: str, kernel: str, commands, n_cu: int = 256,
                      n_xcd: int = 8, min_us: float = 0.0) -> dict:
    """Mean per dispatch of every counter of the matching kernel over the
    given databases (one per counter pass), with the graphics clock
    (GRBM_GUI_ACTIVE of one XCD over the traced duration) and the matrix-pipe
    busy share (SQ_VALU_MFMA_BUSY_CYCLES over the active cycles x CUs x 4
    SIMDs).  With min_us, dispatches shorter than that are left out (they
    need the kernel trace of the same run)."""
    vals, durs = {}, []
    for db in dbs:
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, dispatch_id, counter_name, value "
                           "from counters_collection").fetchall()
        d = kernel_durations(db, kernel)
        if min_us > 0:
            d = {k: v for k, v in d.items() if v >= min_us * 1e3}
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        for kn, did, cn, v in rows:
            if kernel in kn and (min_us <= 0 or did in d):
                per[cn][did] += v
        for cn, by in per.items():
            vals[cn] = sum(by.values()) / len(by)
            if "GRBM_GUI_ACTIVE" == cn and d:
                clk = [by[k] / d[k] for k in by if k in d and d[k] > 0]
                vals.setdefault("_clock_ghz", [])
                vals["_clock_ghz"] += clk
        durs += list(d.values())
    derived = {}
    # GRBM_GUI_ACTIVE is returned per XCD (8 on MI355X) and summed here
    if vals.get("_clock_ghz"):
        derived["graphics clock over the kernel (GHz)"] = (
            sum(vals["_clock_ghz"]) / len(vals["_clock_ghz"]) / n_xcd)
    vals.pop("_clock_ghz", None)
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "GRBM_GUI_ACTIVE" in vals:
        active = vals["GRBM_GUI_ACTIVE"] / n_xcd
        derived["matrix pipe busy share (per SIMD)"] = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (
            active * n_cu * 4)
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in vals:
            derived["matrix and vector issue overlapping (share of cycles, per SIMD)"] = (
                vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / (active * n_cu * 4))
    if durs:
        derived["mean traced duration (us)"] = sum(durs) / len(durs) / 1e3
    lines = [f"# Hardware counters: {os.path.basename(out_md)}", "",
             f"Kernel: `{kernel}` (mean per dispatch; counters summed over their instances).",
             "", "Commands (run from the repository root on one MI355X):", ""]
    for c in commands:
        lines += ["```", c, "```", ""]
    lines += ["| counter | mean per dispatch |", "|---|---:|"]
    for k in sorted(vals):
        lines.append(f"| `{k}` | {vals[k]:.6g} |")
    lines += ["", "| derived | value |", "|---|---:|"]
    for k, v in derived.items():
        lines.append(f"| {k} | {v:.4g} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return {"counters": vals, "derived": derived}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s1 = sub.add_parser("stats")
    s1.add_argument("db")
    s1.add_argument("out")
    s1.add_argument("--command", required=True)
    s2 = sub.add_parser("traffic")
    s2.add_argument("fetch_db")
    s2.add_argument("write_db")
    s2.add_argument("out")
    s2.add_argument("--copy-bytes", type=float, required=True)
    s2.add_argument("--kernel", default="lse_mfma_kernel")
    s2.add_argument("--copy-kernel", default="elementwise")
    s2.add_argument("--source", default="fs_lse.hip", help="kernel source file under csrc/")
    s2.add_argument("--command-fetch", required=True)
    s2.add_argument("--command-write", required=True)
    s3 = sub.add_parser("counters")
    s3.add_argument("out")
    s3.add_argument("--db", action="append", required=True)
    s3.add_argument("--kernel", default="lse_mfma_kernel")
    s3.add_argument("--command", action="append", required=True)
    s3.add_argument("--min-us", type=float, default=0.0,
                    help="leave out dispatches shorter than this (needs the kernel trace)")
    a = ap.parse_args(argv)
    if a.cmd == "counters":
        print(json.dumps(write_counters_md(a.db, a.out, a.kernel, a.command,
                                           min_us=a.min_us), indent=1))
        return 0
    if a.cmd == "stats":
        write_stats_md(a.db, a.out, a.command)
        print(a.out)
    else:
        rec = write_traffic(a.fetch_db, a.write_db, a.out, a.copy_bytes, a.kernel, a.copy_kernel,
                            {"fetch": a.command_fetch, "write": a.command_write}, a.source)
        print(json.dumps(rec, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
