"""Summaries of rocprofv3 output for the library's kernels.

The benchmark quotes two kinds of per-kernel evidence, both kept as short
text records under ``profiles/``:

* kernel time -- ``rocprofv3 --kernel-trace --stats --output-format csv``
  writes ``*_kernel_stats.csv``; :func:`kernel_stats_md` turns it into a
  markdown table;
* hardware counters -- ``rocprofv3 --pmc ... --output-format csv`` writes
  ``*_counter_collection.csv``; :func:`counter_means` averages each counter
  per dispatch of each kernel, and :func:`traffic_record` turns TCC
  FETCH_SIZE / WRITE_SIZE runs into HBM bytes per launch, scaled by what the
  same counters read for a device-to-device copy of known size.

Every record carries the hash of the sources its kernels are built from
(:func:`source_sha`), so a reader can tell whether the figures still
describe the code.

Command line (from the repository root)::

  python -m bit_nf4_quantized_14_amd.profiling stats <dir> --title T --cmd C
  python -m bit_nf4_quantized_14_amd.profiling counters <dir> [<dir> ...]
  python -m bit_nf4_quantized_14_amd.profiling traffic --fetch <dir> \\
      --write <dir> [--copy-bytes N] [--merge profiles/hbm_traffic.json]
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")

# Sources that shape every launch: the shared device and host headers, the
# planning code (tile, split and slice choices, workspace layouts) and the
# entry points that pick the launches.
COMMON_SOURCES = ("qn_device.h", "qn_host.h", "qn_internal.h", "plan.cpp",
                  "linear.hip")
# kernel name prefix -> the source that defines its body
KERNEL_SOURCES = (("k_gemm", "gemm.hip"), ("k_fwd_gemm", "gemm.hip"),
                  ("k_bwd_dx_gemm", "gemm.hip"), ("k_rank", "rank.hip"),
                  ("k_dequant", "codec.hip"), ("k_quantize", "codec.hip"),
                  ("k_skinny", "skinny.hip"), ("k_merge", "merge.hip"),
                  ("k_adamw8", "adamw.hip"))

COPY_BYTES = 256 << 20   # bench.py --calibrate-copy: one 256 MiB copy


def source_sha(kernel: str) -> str | None:
    """sha256[:16] over the common sources and the kernel's own source, or
    None for a kernel this library does not define."""
    for prefix, fname in KERNEL_SOURCES:
        if kernel.startswith(prefix):
            h = hashlib.sha256()
            for f in COMMON_SOURCES + (fname,):
                with open(os.path.join(CSRC, f), "rb") as fh:
                    h.update(fh.read())
            return h.hexdigest()[:16]
    return None


def _find(root: str, suffix: str) -> list[str]:
    return sorted(glob.glob(os.path.join(root, "**", "*" + suffix),
                            recursive=True))


def short_name(name: str) -> str:
    """Kernel name without the return type, the anonymous-namespace prefixes
    and the argument list: ``void (anonymous namespace)::k_gemm<256, 256,
    ...>(...)`` -> ``k_gemm<256, 256, ...>``."""
    n = name.replace("(anonymous namespace)::", "").strip()
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i].strip()
    return n


def kernel_stats(root: str) -> list[dict]:
    """Rows of the kernel_stats.csv files under `root`: name, calls, avg /
    min / max microseconds, percentage of the traced kernel time."""
    rows = []
    for path in _find(root, "kernel_stats.csv"):
        with open(path, newline="") as fh:
            for r in csv.DictReader(fh):
                rows.append({
                    "name": short_name(r["Name"]),
                    "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3,
                    "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3,
                    "pct": float(r["Percentage"]),
                })
    return rows


def kernel_stats_md(root: str, title: str, command: str, note: str = "") -> str:
    rows = kernel_stats(root)
    lines = [f"# Kernel time: {title}", "",
             "Command (from the repository root, after "
             "`cd /tmp && export TMPDIR=/tmp`):", "", "```", command, "```", ""]
    if note:
        lines += [note, ""]
    lines += ["| kernel | calls | avg us | min us | max us | total % |",
              "|---|---:|---:|---:|---:|---:|"]
    for r in sorted(rows, key=lambda r: -r["pct"]):
        lines.append(f"| {r['name']} | {r['calls']} | {r['avg_us']:.1f} | "
                     f"{r['min_us']:.1f} | {r['max_us']:.1f} | {r['pct']:.1f} |")
    shas = sorted({(r["name"], source_sha(r["name"])) for r in rows
                   if source_sha(r["name"])})
    lines += ["", "Kernel source sha256[:16] (common sources + the kernel's "
              ".hip) at measurement: " +
              "; ".join(f"{n}: `{h}`" for n, h in shas)]
    return "\n".join(lines) + "\n"


def counter_means(roots: list[str]) -> dict[str, dict[str, float]]:
    """{kernel: {counter: mean value per dispatch}} over the
    counter_collection.csv files under `roots`."""
    acc = defaultdict(lambda: defaultdict(list))
    for root in roots:
        for path in _find(root, "counter_collection.csv"):
            with open(path, newline="") as fh:
                per = defaultdict(float)   # (dispatch, kernel, counter) sums
                for r in csv.DictReader(fh):
                    key = (r["Dispatch_Id"], short_name(r["Kernel_Name"]),
                           r["Counter_Name"])
                    per[key] += float(r["Counter_Value"])
            for (_, kern, cname), v in per.items():
                acc[kern][cname].append(v)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()}
            for k, cs in acc.items()}


def traffic_record(fetch_root: str, write_root: str,
                   copy_bytes: int = COPY_BYTES) -> dict:
    """HBM bytes per launch from a FETCH_SIZE run and a WRITE_SIZE run (KiB
    per dispatch), each scaled by the factor that makes the copy kernel of
    the same run read and write `copy_bytes` bytes."""
    fetch = counter_means([fetch_root])
    write = counter_means([write_root])

    def copy_value(means, cname):
        vals = [c[cname] for k, c in means.items()
                if cname in c and ("copy" in k.lower() or "Copy" in k)]
        return max(vals) if vals else None

    fc, wc = copy_value(fetch, "FETCH_SIZE"), copy_value(write, "WRITE_SIZE")
    fscale = copy_bytes / (fc * 1024.0) if fc else 1.0
    wscale = copy_bytes / (wc * 1024.0) if wc else 1.0
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        sha = source_sha(k)
        if sha is None or "FETCH_SIZE" not in fetch.get(k, {}) or \
                "WRITE_SIZE" not in write.get(k, {}):
            continue
        kernels[k] = {
            "read_bytes": int(fetch[k]["FETCH_SIZE"] * 1024 * fscale),
            "write_bytes": int(write[k]["WRITE_SIZE"] * 1024 * wscale),
            "fetch_kib_raw": fetch[k]["FETCH_SIZE"],
            "write_kib_raw": write[k]["WRITE_SIZE"],
            "source_sha256_16": sha,
        }
    return {"calibration": {"copy_bytes": copy_bytes, "fetch_scale": fscale,
                            "write_scale": wscale,
                            "copy_fetch_kib": fc, "copy_write_kib": wc},
            "kernels": kernels}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("root")
    a.add_argument("--title", required=True)
    a.add_argument("--cmd", required=True, dest="command")
    a.add_argument("--note", default="")
    c = sub.add_parser("counters")
    c.add_argument("roots", nargs="+")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, default=COPY_BYTES)
    t.add_argument("--merge", help="JSON record to update in place")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        sys.stdout.write(kernel_stats_md(args.root, args.title, args.command,
                                         args.note))
    elif args.cmd == "counters":
        json.dump(counter_means(args.roots), sys.stdout, indent=1)
        sys.stdout.write("\n")
    else:
        rec = traffic_record(args.fetch, args.write, args.copy_bytes)
        if args.merge:
            old = {}
            if os.path.exists(args.merge):
                old = json.load(open(args.merge))
            kernels = dict(old.get("kernels", {}))
            kernels.update(rec["kernels"])
            rec = {"calibration": rec["calibration"], "kernels": kernels}
            with open(args.merge, "w") as fh:
                json.dump(rec, fh, indent=1)
                fh.write("\n")
        else:
            json.dump(rec, sys.stdout, indent=1)
            sys.stdout.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
