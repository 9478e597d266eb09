"""Summaries of rocprofv3 databases (rocpd SQLite) for the solver's kernels.

    python -m streaming_sinkhorn_solver_amd.profiling stats DB OUT.md --command "..."
    python -m streaming_sinkhorn_solver_amd.profiling traffic FETCH_DB WRITE_DB OUT.json \
        --copy-bytes B --kernel lse_mfma_kernel --source fs_lse.hip \
        --command-fetch "..." --command-write "..."

`stats` tabulates kernel-trace durations (calls, mean, min, max, share).
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
    a = ap.parse_args(argv)
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
