"""Summaries of rocprofv3 output for the libsas kernels (text, a few KB).

Two summaries are made, both as Markdown:

* ``stats``: the per-kernel table of a ``rocprofv3 --kernel-trace --stats
  --output-format csv`` run (calls, total, average, min, max in microseconds).
* ``traffic``: HBM bytes per dispatch from two ``rocprofv3 --pmc`` runs, one
  with ``FETCH_SIZE`` and one with ``WRITE_SIZE`` (both in KiB per dispatch).
  Each counter is scaled by what it reads for a plain device copy of known
  size run in the same process (the largest ``__amd_rocclr_copyBuffer``
  dispatch), so ``bytes = counter_KiB * 1024 * known_bytes / copy_counter_bytes``.
  The summary ends with a JSON block (per-kernel scaled bytes and the SHA-256
  of the kernel sources) that ``bench.py`` reads to fill ``roofline.traffic``;
  once a source file changes the hashes no longer match and the traffic is
  reported as unknown.

Usage::

    python -m gated_block_sparse_amd.profsum stats DIR --cmd "..." --title "..."
    python -m gated_block_sparse_amd.profsum traffic FETCH_DIR WRITE_DIR \
        --copy-bytes 1073741824 --cmd-fetch "..." --cmd-write "..." --title "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def short_name(name: str) -> str:
    """Kernel name without its argument list (templates kept)."""
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            name = name[:i]
            break
    return re.sub(r"^void ", "", name).strip()


def source_hashes() -> dict:
    """SHA-256 of every kernel source and header of the library."""
    out = {}
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if path.endswith((".hip", ".h")):
            with open(path, "rb") as f:
                out[os.path.basename(path)] = hashlib.sha256(f.read()).hexdigest()
    return out


def _one(pattern: str, where: str) -> str:
    hits = sorted(glob.glob(os.path.join(where, "**", pattern), recursive=True))
    if not hits:
        raise SystemExit(f"no {pattern} under {where}")
    return hits[0]


def stats(args) -> str:
    path = _one("*kernel_stats.csv", args.dir)
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# {args.title}", "", "Command (run from /tmp, repository at $R):", "", "```",
             args.cmd, "```", "",
             "| kernel | calls | total us | avg us | min us | max us | % |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append("| `{}` | {} | {:.1f} | {:.3f} | {:.3f} | {:.3f} | {:.2f} |".format(
            short_name(r["Name"]), r["Calls"], float(r["TotalDurationNs"]) / 1e3,
            float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["Percentage"])))
    return "\n".join(lines) + "\n"


def _counter(path: str, name: str):
    per = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == name:
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def traffic(args) -> str:
    fetch = _counter(_one("*counter_collection.csv", args.fetch_dir), "FETCH_SIZE")
    write = _counter(_one("*counter_collection.csv", args.write_dir), "WRITE_SIZE")
    if COPY_KERNEL not in fetch or COPY_KERNEL not in write:
        raise SystemExit("no calibration copy dispatch in the PMC runs")
    cf = max(fetch[COPY_KERNEL]) * 1024.0
    cw = max(write[COPY_KERNEL]) * 1024.0
    f_scale, w_scale = args.copy_bytes / cf, args.copy_bytes / cw
    kern = {}
    for name in sorted(set(fetch) | set(write)):
        if "sas::" not in name:
            continue
        fv, wv = fetch.get(name, []), write.get(name, [])
        kern[short_name(name)] = {
            "dispatches": max(len(fv), len(wv)),
            "fetch_kib": round(sum(fv) / max(len(fv), 1), 2),
            "write_kib": round(sum(wv) / max(len(wv), 1), 2),
            "fetch_bytes": round(sum(fv) / max(len(fv), 1) * 1024.0 * f_scale),
            "write_bytes": round(sum(wv) / max(len(wv), 1) * 1024.0 * w_scale),
        }
    lines = [f"# {args.title}", "",
             "Commands (run from /tmp, repository at $R):", "", "```", args.cmd_fetch,
             args.cmd_write, "```", "",
             f"Calibration: a plain device copy of {args.copy_bytes} bytes read "
             f"FETCH_SIZE = {cf / 1024:.0f} KiB and WRITE_SIZE = {cw / 1024:.0f} KiB, "
             f"so FETCH_SIZE is scaled by {f_scale:.3f} and WRITE_SIZE by {w_scale:.3f}.", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read bytes | HBM write bytes |",
             "|---|---:|---:|---:|---:|---:|"]
    for n, v in kern.items():
        lines.append(f"| `{n}` | {v['dispatches']} | {v['fetch_kib']} | {v['write_kib']} | "
                     f"{v['fetch_bytes']} | {v['write_bytes']} |")
    blob = {"copy_bytes": args.copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale,
            "kernels": kern, "sources_sha256": source_hashes()}
    lines += ["", "Per-dispatch bytes and source hashes (read by bench.py):", "", "```json",
              json.dumps(blob, indent=1), "```"]
    return "\n".join(lines) + "\n"


def load_traffic(path: str, sources=None):
    """The JSON block of a traffic summary, or None when the file is missing
    or a kernel source changed since the counters were taken (every source,
    or only the named files when `sources` is given)."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    blob = json.loads(m.group(1))
    then, now = blob.get("sources_sha256", {}), source_hashes()
    names = list(now) if sources is None else list(sources)
    if any(then.get(n) is None or then.get(n) != now.get(n) for n in names):
        return None
    return blob


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--cmd", required=True)
    a.add_argument("--title", required=True)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    b.add_argument("--title", required=True)
    args = ap.parse_args(argv)
    sys.stdout.write(stats(args) if args.what == "stats" else traffic(args))


if __name__ == "__main__":
    main()
