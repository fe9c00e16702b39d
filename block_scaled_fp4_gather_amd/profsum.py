"""Summaries of rocprofv3 runs for the profiles/ folder, and their lookup.

    python -m block_scaled_fp4_gather_amd.profsum WORKLOAD TRACE_DB FETCH_CSV WRITE_CSV \
        COPY_FETCH_CSV COPY_WRITE_CSV "COMMAND"

reads one kernel-trace database (``--kernel-trace --stats``), two counter
runs of the benchmark (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``) and the
same two counters for the benchmark's copy probe (a device copy of 256 MiB
each way), and writes ``profiles/<kernel>.<workload>.md`` for each layer
kernel (decode: fc1_kernel, fc2_kernel; grouped: fc1_gemm, fc2_gemm, or with
MXFP8 activations fc1_gemm_a8, fc2_gemm_a8 and mxfp8_quantize, and the
routing and combine kernels).  Each summary ends with a JSON block that bench.py reads back; the
counters there are tied to a hash of the kernel's HIP sources so that a
summary taken before a change to that kernel is not used after it.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sqlite3
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 * 1024 * 1024  # bench.py --copy-probe: bytes read and written per dispatch
# (more specific names first: a kernel is named by the first entry its symbol contains)
KERNELS = ("fc1_kernel", "fc2_kernel", "fc1_gemm_a8", "fc2_gemm_a8", "mxfp8_quantize", "fc1_gemm", "fc2_gemm",
           "route_one", "route_count", "route_place", "route_zero", "combine")


# HIP sources each kernel is built from: a summary stays valid while their
# code (comments and blank space aside) is unchanged.
_DECODE_SRC = ("decode_path.hip", "decode_path.h", "decode.h", "act.h", "layout.h")
_GROUPED_SRC = ("prefill.hip", "prefill.h", "gemm_util.h", "gemm_planes.h", "mxfp8.h", "decode.h", "act.h",
                "layout.h")
_A8_SRC = ("prefill_a8.hip", "prefill.h", "gemm_util.h", "gemm_planes.h", "mxfp8.h", "act.h", "layout.h")
SOURCES = {"fc1_kernel": _DECODE_SRC, "fc2_kernel": _DECODE_SRC, "fc1_gemm": _GROUPED_SRC,
           "fc2_gemm": _GROUPED_SRC, "route_one": _GROUPED_SRC, "route_count": _GROUPED_SRC,
           "route_place": _GROUPED_SRC, "route_zero": _GROUPED_SRC, "combine": _GROUPED_SRC,
           "fc1_gemm_a8": _A8_SRC, "fc2_gemm_a8": _A8_SRC, "mxfp8_quantize": ("mxfp8.hip", "mxfp8.h")}


def _code(text: str) -> str:
    """Source text without comments, with runs of blank space collapsed."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif text[i] == '"':  # string literal, copied whole
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for name in sorted(SOURCES[kernel]):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code(f.read()).encode())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    for k in KERNELS:
        if k in name:
            return k
    return name.split("(")[0][-48:]


def trace_stats(db: str) -> dict:
    c = sqlite3.connect(db)
    d: dict = {}
    for name, dur in c.execute("select name, duration from kernels"):
        d.setdefault(_short(name), []).append(dur / 1000.0)
    return {k: {"calls": len(v), "mean_us": statistics.mean(v), "median_us": statistics.median(v),
                "min_us": min(v)} for k, v in d.items()}


def counter(path: str, name: str) -> dict:
    vals: dict = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == name:
                vals.setdefault(_short(row["Kernel_Name"]), []).append(float(row["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def copy_reference(path: str, name: str) -> float:
    """Counter value (KiB per dispatch) of the 256 MiB copy kernel."""
    vals = counter(path, name)
    big = [v for v in vals.values() if v > 1024]
    if not big:
        raise ValueError(f"no copy dispatch with {name} in {path}")
    return max(big)


def write(workload: str, trace_db: str, fetch_csv: str, write_csv: str, copy_fetch: str,
          copy_write: str, command: str) -> list[str]:
    stats = trace_stats(trace_db)
    fetch = counter(fetch_csv, "FETCH_SIZE")
    wsize = counter(write_csv, "WRITE_SIZE")
    ref_f = copy_reference(copy_fetch, "FETCH_SIZE")
    ref_w = copy_reference(copy_write, "WRITE_SIZE")
    f_scale = COPY_BYTES / 1024 / ref_f  # true bytes per counted byte
    w_scale = COPY_BYTES / 1024 / ref_w
    out = []
    os.makedirs(PROFILES, exist_ok=True)
    for k in KERNELS:
        if k not in stats:
            continue
        rec = {
            "kernel": k, "workload": workload, "source_hash": source_hash(k),
            "duration_us": {kk: round(v, 3) for kk, v in stats[k].items() if kk != "calls"},
            "dispatches": stats[k]["calls"],
            "FETCH_SIZE_KiB": round(fetch.get(k, float("nan")), 1),
            "WRITE_SIZE_KiB": round(wsize.get(k, float("nan")), 1),
            "copy_reference_KiB": {"FETCH_SIZE": round(ref_f, 1), "WRITE_SIZE": round(ref_w, 1),
                                   "true_KiB_each_way": COPY_BYTES // 1024},
            "scale": {"fetch": round(f_scale, 4), "write": round(w_scale, 4)},
            "hbm_bytes_per_dispatch": round((fetch.get(k, 0.0) * f_scale + wsize.get(k, 0.0) * w_scale) * 1024),
        }
        others = {kk: {"calls": v["calls"], "mean_us": round(v["mean_us"], 3)} for kk, v in stats.items()}
        path = os.path.join(PROFILES, f"{k}.{workload}.md")
        with open(path, "w") as f:
            f.write(f"# {k} on {workload} (MI355X, rocprofv3)\n\n")
            f.write("Commands (run from the repository root; the counter runs each use one counter):\n\n")
            f.write("```\n" + command.strip() + "\n```\n\n")
            f.write("| quantity | value |\n|---|---|\n")
            f.write(f"| dispatches traced | {rec['dispatches']} |\n")
            f.write(f"| duration mean / median / min (us) | {rec['duration_us']['mean_us']} / "
                    f"{rec['duration_us']['median_us']} / {rec['duration_us']['min_us']} |\n")
            f.write(f"| FETCH_SIZE per dispatch (KiB, raw) | {rec['FETCH_SIZE_KiB']} |\n")
            f.write(f"| WRITE_SIZE per dispatch (KiB, raw) | {rec['WRITE_SIZE_KiB']} |\n")
            f.write(f"| copy kernel, 256 MiB each way: FETCH_SIZE / WRITE_SIZE (KiB) | {round(ref_f, 1)} / "
                    f"{round(ref_w, 1)} |\n")
            f.write(f"| scale (true / counted): fetch, write | {rec['scale']['fetch']}, {rec['scale']['write']} |\n")
            f.write(f"| HBM bytes per dispatch (scaled) | {rec['hbm_bytes_per_dispatch']} |\n\n")
            f.write("All kernels in the trace (calls, mean us):\n\n")
            for kk, v in sorted(others.items(), key=lambda kv: -kv[1]["calls"] * kv[1]["mean_us"]):
                f.write(f"- {kk}: {v['calls']} calls, {v['mean_us']} us\n")
            f.write("\n```json\n" + json.dumps(rec, indent=1) + "\n```\n")
        out.append(path)
    return out


def lookup(kernel: str, workload: str) -> dict | None:
    """The recorded counters of a kernel on a workload, if the HIP sources
    are unchanged since they were taken."""
    path = os.path.join(PROFILES, f"{kernel}.{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        rec = json.loads(text[text.rindex("```json") + 7:text.rindex("```")])
    except ValueError:
        return None
    return rec if rec.get("source_hash") == source_hash(kernel) else None


if __name__ == "__main__":
    if len(sys.argv) != 8:
        sys.exit(__doc__)
    for p in write(*sys.argv[1:8]):
        print(p)
