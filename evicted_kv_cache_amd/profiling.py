"""Summaries of rocprofv3 output for the kernels of libkvq.

Reads the CSV files rocprofv3 writes (``--kernel-trace --stats`` and
``--pmc``) and prints short text summaries: per-kernel average durations,
per-dispatch counter averages, and HBM traffic per launch from the
FETCH_SIZE / WRITE_SIZE counters scaled by what the same counters read for a
device copy of known size.

  python -m evicted_kv_cache_amd.profiling stats  <kernel_stats.csv> --cmd "<command>"
  python -m evicted_kv_cache_amd.profiling counters <counter_collection.csv> [...] --cmd "<command>"
  python -m evicted_kv_cache_amd.profiling traffic --fetch F.csv --write W.csv \
      --copy-fetch CF.csv --copy-write CW.csv --copy-bytes N --kernel decode_mfma \
      [--source file.hip] [--cmd "<command>" ...]

Host-side tooling only: it runs nothing on the GPU.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import sys


def short_name(name: str, width: int = 90) -> str:
    """Kernel name without the namespace prefix and argument list."""
    n = name.replace("kvq::(anonymous namespace)::", "").replace("at::native::", "")
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            n = n[:i]
            break
    return n if len(n) <= width else n[: width - 3] + "..."


def kernel_stats(path: str):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Name"], "calls": int(r["Calls"]),
                         "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                         "max_us": float(r["MaxNs"]) / 1e3, "pct": float(r["Percentage"])})
    return rows


def counter_rows(path: str):
    """{(kernel name, counter): [value per dispatch]}"""
    out = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            out[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return out


def counter_avg(path: str, counter: str, kernel_prefix: str, min_value: float = 0.0):
    """Average of `counter` over dispatches of kernels whose short name starts
    with kernel_prefix (dispatches reading below min_value are skipped)."""
    vals = []
    for (name, c), v in counter_rows(path).items():
        if c == counter and short_name(name, 10**6).startswith(kernel_prefix):
            vals += [x for x in v if x >= min_value]
    if not vals:
        raise SystemExit(f"no {counter} dispatches of '{kernel_prefix}' in {path}")
    return sum(vals) / len(vals), len(vals)


def sha16(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cmd_stats(a):
    rows = kernel_stats(a.csv)
    print(f"# rocprofv3 kernel statistics\n\nCommand: `{a.cmd}`\n")
    print("| kernel | calls | avg us | min us | max us | % time |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in rows:
        print(f"| `{short_name(r['name'])}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
              f"{r['max_us']:.2f} | {r['pct']:.2f} |")


def cmd_counters(a):
    print(f"# rocprofv3 counters (average per dispatch)\n")
    for c in a.cmd:
        print(f"Command: `{c}`  ")
    print("\n| kernel | counter | dispatches | average |")
    print("|---|---|---:|---:|")
    for path in a.csv:
        for (name, c), v in sorted(counter_rows(path).items()):
            if a.kernel and not any(short_name(name, 10**6).startswith(k) for k in a.kernel):
                continue
            print(f"| `{short_name(name)}` | {c} | {len(v)} | {sum(v) / len(v):.6g} |")


def cmd_traffic(a):
    cf, ncf = counter_avg(a.copy_fetch, "FETCH_SIZE", a.copy_kernel, a.copy_bytes / 1024 / 8)
    cw, ncw = counter_avg(a.copy_write, "WRITE_SIZE", a.copy_kernel, a.copy_bytes / 1024 / 8)
    f_factor = a.copy_bytes / (cf * 1024)
    w_factor = a.copy_bytes / (cw * 1024)
    out = {"copy_kernel": a.copy_kernel, "copy_bytes_each_way": a.copy_bytes,
           "copy_fetch_kib": round(cf, 3), "copy_write_kib": round(cw, 3),
           "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4), "kernels": {}}
    for k in a.kernel:
        f, nf = counter_avg(a.fetch, "FETCH_SIZE", k)
        w, nw = counter_avg(a.write, "WRITE_SIZE", k)
        out["kernels"][k] = {"fetch_kib_per_dispatch": round(f, 3), "write_kib_per_dispatch": round(w, 3),
                             "dispatches": [nf, nw],
                             "bytes_per_launch": int(round(f * 1024 * f_factor + w * 1024 * w_factor))}
    if a.source:
        out["source_sha256_16"] = sha16(a.source)
        out["source"] = a.source
    out["commands"] = a.cmd
    if len(a.kernel) == 1:
        out["bytes_per_launch"] = out["kernels"][a.kernel[0]]["bytes_per_launch"]
    json.dump(out, sys.stdout, indent=1)
    print()


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m evicted_kv_cache_amd.profiling")
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", action="append", default=[])
    c.add_argument("--cmd", action="append", default=[])
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--copy-kernel", default="__amd_rocclr_copyBuffer")
    t.add_argument("--kernel", action="append", required=True)
    t.add_argument("--source")
    t.add_argument("--cmd", action="append", default=[])
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "counters": cmd_counters, "traffic": cmd_traffic}[a.what](a)


if __name__ == "__main__":
    main()
