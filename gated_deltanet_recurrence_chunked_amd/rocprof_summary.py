"""Turns rocprofv3 CSV output into the short text summaries kept under profiles/.

  kernels  KTRACE_DIR OUT.txt "COMMAND"
      per (kernel, grid size) calls / average / median / min / max duration from
      <KTRACE_DIR>/*kernel_trace.csv
  traffic  FETCH_DIR WRITE_DIR OUT.json "COMMAND"
      FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of every library kernel, scaled by what the
      same counters read for the 1 GiB measurement copy the benchmark runs (the factor turns
      counter KiB into bytes that cross HBM)
  mfma     PMC_DIR OUT.json "COMMAND"
      bf16 / fp32 matrix-core flops and matrix-core busy share per dispatch of every library
      kernel

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
# the kernels of one gdn_chunk_prefill call (bf16 y; the states-only scan instantiation that the
# backward runs is another kernel)
PREFILL_KERNELS = ("chunk_prep_kernel<false>", "chunk_scan_fwd_kernel<unsigned short>",
                   "chunk_scan_kernel<unsigned short, false, true>", "chunk_table_kernel")


PREFILL_SOURCES = ("chunk_bf16.hip", "gdn_device.h", "gdn_inverse.h", "gdn_mfma.h")


def prefill_source_sha() -> str:
    """Hash of the chunked-prefill kernel source and the headers it includes: counters are
    void once any of them changes."""
    h = hashlib.sha256()
    for name in PREFILL_SOURCES:
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def source_shas() -> dict:
    """Hash of every library source file: a counter figure of a kernel is void once the file
    that holds it (or a header it includes) changes."""
    out = {}
    for path in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        with open(path, "rb") as f:
            out[os.path.basename(path)] = hashlib.sha256(f.read()).hexdigest()[:16]
    return out


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("gdn::", "").replace("void ", "")
    return name.split("(")[0]


def kernels(ktrace_dir: str, out: str, command: str) -> None:
    """Per (kernel, grid) duration statistics from the kernel trace: one line per workload a
    kernel ran, so launches of different sizes are not averaged together."""
    path = _one(os.path.join(ktrace_dir, "**", "*kernel_trace.csv"))
    per = defaultdict(list)
    for r in csv.DictReader(open(path)):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        per[(r["Kernel_Name"], grid)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in per.values())
    lines = ["# rocprofv3 --kernel-trace summary, per kernel and grid size (threads)",
             f"# command: {command}", "",
             f"{'kernel':64s} {'grid':>9s} {'calls':>6s} {'avg_us':>9s} {'med_us':>9s} "
             f"{'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for (name, grid), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        v = sorted(v)
        lines.append(f"{short(name)[:64]:64s} {grid:9d} {len(v):6d} {sum(v) / len(v):9.2f} "
                     f"{v[len(v) // 2]:9.2f} {v[0]:9.2f} {v[-1]:9.2f} {100 * sum(v) / total:6.2f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter(dir_: str, counter: str):
    """Counter values per dispatch, keyed by kernel name and grid size (one workload each)."""
    path = _one(os.path.join(dir_, "**", "*counter_collection.csv"))
    per = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return per


def _key(k) -> str:
    name, grid = k
    return f"{short(name)} [grid {grid}]"


def _library_kernel(name: str) -> bool:
    """Kernels of libgdn (torch's own kernels and the runtime's blits are left out)."""
    sk = short(name)
    return not (sk.startswith("at::") or sk.startswith("__amd") or "at::native" in name)


def traffic(fetch_dir: str, write_dir: str, out: str, command: str) -> None:
    """FETCH_SIZE and WRITE_SIZE per dispatch of every library kernel, in bytes: the counters'
    KiB scaled by what they read for the 1 GiB measurement copy (stream_kernel, 1 GiB read and
    1 GiB written per dispatch)."""
    res = {"command": command, "kernel_source_sha256": prefill_source_sha(),
           "source_sha256": source_shas(), "kernels": {}}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _counter(d, counter)
        copies = [max(v) for k, v in per.items() if "stream_kernel" in k[0]]
        if not copies:
            raise SystemExit(f"no stream_kernel dispatch among {list(per)}")
        copy_kib = max(copies)
        factor = (COPY_BYTES / 1024.0) / copy_kib
        res[f"copy_{counter}_kib"] = copy_kib
        res[f"{counter}_factor"] = factor
        for k, v in per.items():
            if not _library_kernel(k[0]) or "stream_kernel" in k[0]:
                continue
            e = res["kernels"].setdefault(_key(k), {"dispatches": len(v)})
            e[f"{counter}_kib_per_dispatch"] = sum(v) / len(v)
            e[f"{counter}_bytes"] = sum(v) / len(v) * 1024.0 * factor
    total = 0.0
    for sk, e in res["kernels"].items():
        e["bytes"] = e.get("FETCH_SIZE_bytes", 0.0) + e.get("WRITE_SIZE_bytes", 0.0)
        if sk.split(" [grid")[0] in PREFILL_KERNELS:
            total += e["bytes"]
    res["gdn_chunk_prefill_bytes_per_call"] = total
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


XCC_NUM = 8        # GRBM_GUI_ACTIVE is summed over the 8 XCDs in the counter file
SIMD_NUM = 1024    # 256 CUs x 4 SIMDs


def mfma(pmc_dir: str, out: str, command: str) -> None:
    """Matrix-core counters per dispatch of every library kernel:
      flops_bf16 / flops_f32  SQ_INSTS_VALU_MFMA_MOPS_{BF16,F32} x 512 (the counters count
                              multiply-add work in units of 512 flops);
      mfma_busy_frac          SQ_VALU_MFMA_BUSY_CYCLES over (GRBM_GUI_ACTIVE / XCDs) x SIMDs,
                              the share of SIMD-cycles the matrix cores were busy."""
    res = {"command": command, "kernel_source_sha256": prefill_source_sha(),
           "source_sha256": source_shas(), "kernels": {}}
    cnt = {c: _counter(pmc_dir, c) for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                                "SQ_INSTS_VALU_MFMA_MOPS_F32",
                                                "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")}
    names = set()
    for per in cnt.values():
        names.update(k for k in per if _library_kernel(k[0]))
    total = 0.0
    for k in sorted(names):
        avg = {c: (sum(per[k]) / len(per[k]) if per.get(k) else 0.0) for c, per in cnt.items()}
        gui = avg["GRBM_GUI_ACTIVE"] / XCC_NUM
        e = {"dispatches": len(cnt["GRBM_GUI_ACTIVE"].get(k, [])),
             "flops_bf16": avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0,
             "flops_f32": avg["SQ_INSTS_VALU_MFMA_MOPS_F32"] * 512.0,
             "gui_active_cycles": gui,
             "mfma_busy_frac": (avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * SIMD_NUM)) if gui else None}
        res["kernels"][_key(k)] = e
        if short(k[0]) in PREFILL_KERNELS:
            total += e["flops_bf16"] + e["flops_f32"]
    res["gdn_chunk_prefill_mfma_flops_per_call"] = total
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "kernels":
        kernels(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 6 and sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    elif len(sys.argv) >= 5 and sys.argv[1] == "mfma":
        mfma(sys.argv[2], sys.argv[3], sys.argv[4])
    else:
        print(__doc__)
        sys.exit(2)
