"""Summaries of rocprofv3 CSV output for the library's kernels (a measurement helper; the
committed summaries under profiles/ are written by it).

  python -m sparse_global_attention_block_amd.profsum kernels <dir> [--cmd "..."]
      -> markdown table of the library's kernels from <dir>/*kernel_stats.csv
  python -m sparse_global_attention_block_amd.profsum bytes <fetch_dir> <write_dir>
        <copy_fetch_dir> <copy_write_dir> --workload W --copy-bytes N [--cmd "..."] [--json F]
      -> HBM bytes per dispatch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what
         the same counters read for the library's streaming copy of N bytes
  python -m sparse_global_attention_block_amd.profsum counters <dir> [<dir> ...] [--cmd "..."]
      -> per-kernel derived counters (MfmaUtil, VALUBusy, ...) of the longest dispatch
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))


def short(name: str) -> str:
    """Kernel name without 'void ' and its argument list."""
    name = re.sub(r"^void ", "", name)
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):  # drop the trailing "(Args)" at template depth 0
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    return name[:cut]


def rows(directory: str, pattern: str):
    out = []
    for f in sorted(glob.glob(os.path.join(directory, "**", pattern), recursive=True)):
        with open(f) as fh:
            out += list(csv.DictReader(fh))
    return out


def mine(name: str) -> bool:
    return name.startswith("s3r::")


def kernels(directory: str, cmd: str) -> str:
    stats = [r for r in rows(directory, "*kernel_stats.csv") if mine(short(r["Name"]))]
    total = sum(float(r["TotalDurationNs"]) for r in stats) or 1.0
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["| kernel | calls | avg ms | min ms | max ms | % of the library's GPU time |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                     f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.1f} |")
    return f"Command:\n\n```\n{cmd}\n```\n\n" + "\n".join(lines) + "\n"


def per_kernel(directory: str, counter: str):
    """{kernel: [value per dispatch]} of one counter."""
    vals = defaultdict(list)
    for r in rows(directory, "*counter_collection.csv"):
        if r["Counter_Name"] == counter:
            vals[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return vals


def source_sha256() -> str:
    h = hashlib.sha256()
    for f in ("s3r_cmp.hip", "s3r_common.hpp"):
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def hbm_bytes(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, workload, copy_bytes, cmd):
    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    cf = per_kernel(copy_fetch_dir, "FETCH_SIZE").get("s3r::calib_copy_kernel")
    cw = per_kernel(copy_write_dir, "WRITE_SIZE").get("s3r::calib_copy_kernel")
    if not cf or not cw:
        raise SystemExit("no s3r::calib_copy_kernel dispatch in the calibration runs")
    fscale = copy_bytes / (max(cf) * 1024.0)
    wscale = copy_bytes / (max(cw) * 1024.0)
    rec = {"workload": workload, "fetch_scale": fscale, "write_scale": wscale,
           "cmp_fused_source_sha256": source_sha256(), "kernels": {}}
    lines = [f"Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two separate rocprofv3 "
             f"runs, each scaled by what the same counter reads for the library's streaming copy "
             f"of {copy_bytes} bytes (`s3r::calib_copy_kernel`, which reads and writes that many): "
             f"FETCH_SIZE scale {fscale:.3f}, WRITE_SIZE scale {wscale:.3f}. Mean over dispatches.",
             "", f"Commands (from /tmp, TMPDIR=/tmp; one run per counter):", "", "```", cmd, "```",
             "", "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB (scaled) | "
                 "written GB (scaled) |", "|---|---|---|---|---|---|"]
    names = sorted((k for k in fetch if mine(k)), key=lambda k: -max(fetch[k]))
    for k in names:
        f = sum(fetch[k]) / len(fetch[k])
        wv = write.get(k, [0.0])
        wr = sum(wv) / len(wv)
        rb, wb = f * 1024 * fscale, wr * 1024 * wscale
        rec["kernels"][k] = {"read_bytes": rb, "write_bytes": wb, "dispatches": len(fetch[k])}
        lines.append(f"| `{k}` | {len(fetch[k])} | {f:.4g} | {wr:.4g} | {rb / 1e9:.2f} | "
                     f"{wb / 1e9:.2f} |")
    return rec, "\n".join(lines) + "\n"


def counters(dirs, cmd):
    """Derived counters per kernel: the value of the kernel's longest-running dispatch (by the
    dispatch timestamps of the same rows)."""
    table = defaultdict(dict)
    names = []
    for d in dirs:
        best = {}
        for r in rows(d, "*counter_collection.csv"):
            k = short(r["Kernel_Name"])
            if not mine(k):
                continue
            dur = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            key = (k, r["Counter_Name"])
            if key not in best or dur > best[key][0]:
                best[key] = (dur, float(r["Counter_Value"]))
        for (k, c), (dur, v) in best.items():
            table[k][c] = v
            table[k]["_ms"] = max(table[k].get("_ms", 0.0), dur / 1e6)
            if c not in names:
                names.append(c)
    lines = ["| kernel | longest dispatch ms | " + " | ".join(names) + " |",
             "|---|---|" + "---|" * len(names)]
    for k in sorted(table, key=lambda k: -table[k]["_ms"]):
        lines.append(f"| `{k}` | {table[k]['_ms']:.3f} | " +
                     " | ".join(f"{table[k][c]:.4g}" if c in table[k] else "—" for c in names) +
                     " |")
    return f"Command (one run per counter set):\n\n```\n{cmd}\n```\n\n" + "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["kernels", "bytes", "counters"])
    ap.add_argument("dirs", nargs="+")
    ap.add_argument("--cmd", default="")
    ap.add_argument("--workload", default="")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--json", default=None)
    a = ap.parse_args()
    if a.mode == "kernels":
        print(kernels(a.dirs[0], a.cmd))
    elif a.mode == "bytes":
        rec, md = hbm_bytes(*a.dirs[:4], a.workload, a.copy_bytes, a.cmd)
        print(md)
        if a.json:
            with open(a.json, "w") as fh:
                json.dump(rec, fh, indent=1)
    else:
        print(counters(a.dirs, a.cmd))


if __name__ == "__main__":
    main()
