"""Turns rocprofv3 CSV output into the short text summaries kept under profiles/.

  kernels  KTRACE_DIR OUT.txt "COMMAND"
      per-kernel calls / average / min / max duration from <KTRACE_DIR>/*kernel_stats.csv
  traffic  FETCH_DIR WRITE_DIR OUT.json "COMMAND"
      FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the chunked-prefill kernels, scaled by
      what the same counters read for the plain 1 GiB device copy the benchmark runs with
      --calibrate-copy (the factor turns counter KiB into bytes that cross HBM)

Usage: python -m gated_deltanet_recurrence_chunked_amd.rocprof_summary kernels ...
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30
PREFILL_KERNELS = ("chunk_prep_kernel", "chunk_scan_kernel", "chunk_table_kernel")


PREFILL_SOURCES = ("chunk_bf16.hip", "gdn_device.h", "gdn_inverse.h", "gdn_launch.h")


def prefill_source_sha() -> str:
    """Hash of the chunked-prefill kernel source and the headers it includes: counters are
    void once any of them changes."""
    h = hashlib.sha256()
    for name in PREFILL_SOURCES:
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("gdn::", "").replace("void ", "")
    return name.split("(")[0]


def kernels(ktrace_dir: str, out: str, command: str) -> None:
    path = _one(os.path.join(ktrace_dir, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    lines = [f"# rocprofv3 --kernel-trace --stats summary", f"# command: {command}", "",
             f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{short(r['Name'])[:70]:70s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter(dir_: str, counter: str):
    path = _one(os.path.join(dir_, "**", "*counter_collection.csv"))
    per = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def traffic(fetch_dir: str, write_dir: str, out: str, command: str) -> None:
    res = {"command": command, "kernel_source_sha256": prefill_source_sha(), "kernels": {}}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _counter(d, counter)
        copies = [max(v) for k, v in per.items() if "copyBuffer" in k or "copy" in k.lower()]
        if not copies:
            raise SystemExit(f"no copy kernel among {list(per)}")
        copy_kib = max(copies)
        factor = (COPY_BYTES / 1024.0) / copy_kib
        res[f"copy_{counter}_kib"] = copy_kib
        res[f"{counter}_factor"] = factor
        for k, v in per.items():
            sk = short(k)
            if any(p in sk for p in PREFILL_KERNELS):
                e = res["kernels"].setdefault(sk, {})
                e[f"{counter}_kib_per_dispatch"] = sum(v) / len(v)
                e[f"{counter}_bytes"] = sum(v) / len(v) * 1024.0 * factor
    total = 0.0
    for sk, e in res["kernels"].items():
        e["bytes"] = e.get("FETCH_SIZE_bytes", 0.0) + e.get("WRITE_SIZE_bytes", 0.0)
        total += e["bytes"]
    res["gdn_chunk_prefill_bytes_per_call"] = total
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "kernels":
        kernels(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 6 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    else:
        print(__doc__)
        sys.exit(2)
