"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m speculative_decoding_round_amd.profsum stats  KERNEL_STATS_CSV BENCH_JSON OUT.txt CMD
    python -m speculative_decoding_round_amd.profsum traffic FETCH_CSV WRITE_CSV OUT.txt CMD

`stats` lists the kernels of a `rocprofv3 --kernel-trace --stats` run with their average
duration, marks the LM-head GEMM and puts bench.py's own event-timed average beside it.
`traffic` reads one `--pmc FETCH_SIZE` and one `--pmc WRITE_SIZE` run (KiB per dispatch),
scales both by what the same counter reads for the plain 1 GiB device copy that
`bench.py --copy-calibration-mb 1024` adds, and records the HBM bytes per LM-head launch
with a hash of the GEMM kernel source, so bench.py can tell when they went stale.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
LM_HEAD_KERNEL = re.compile(r"k_gemm_ring<1, 8, 4, false>")   # the LM head (one 16-row tile of rows)


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h"):
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    m = re.search(r"(k_[a-z_0-9]+)(<[^()]*>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else name[:60]


def stats(csv_path, bench_json, out, cmd):
    rows = list(csv.DictReader(open(csv_path)))
    bench = json.loads(open(bench_json).read().strip().splitlines()[-1])
    lines = [f"# rocprofv3 kernel stats, {bench['config']['workload']}", f"command: {cmd}", "",
             f"{'calls':>6} {'avg_us':>10} {'total_%':>8}  kernel"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:24]:
        mark = "  <- LM head" if LM_HEAD_KERNEL.search(r["Name"]) else ""
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['Percentage']):8.2f}  {_short(r['Name'])}{mark}")
    lm = [r for r in rows if LM_HEAD_KERNEL.search(r["Name"])]
    if lm:
        lines += ["", f"LM-head GEMM average (rocprofv3): {float(lm[0]['AverageNs']) / 1e3:.2f} us",
                  f"LM-head GEMM average (bench.py HIP events, same run): "
                  f"{bench['roofline']['avg_launch_us']:.2f} us",
                  f"bench ms_per_step under the profiler: {bench['ms_per_step']}"]
    open(out, "w").write("\n".join(lines) + "\n")


def _per_kernel(csv_path):
    agg = defaultdict(list)
    for r in csv.DictReader(open(csv_path)):
        agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def traffic(fetch_csv, write_csv, out, cmd):
    f, w = _per_kernel(fetch_csv), _per_kernel(write_csv)
    copy = [k for k in f if "copyBuffer" in k]
    known = 1 << 20                                     # KiB moved each way by the 1 GiB copy
    f_copy = max(max(f[k]) for k in copy)
    w_copy = max(max(w[k]) for k in copy)
    ff, wf = known / f_copy, known / w_copy
    lm = [k for k in f if LM_HEAD_KERNEL.search(k)][0]
    fetch = sum(f[lm]) / len(f[lm]) * ff * 1024
    write = sum(w[lm]) / len(w[lm]) * wf * 1024
    lines = ["# HBM traffic of the LM-head GEMM (rocprofv3 --pmc), llama8b workload",
             f"command_fetch: {cmd.format(counter='FETCH_SIZE')}",
             f"command_write: {cmd.format(counter='WRITE_SIZE')}",
             f"copy_calibration: 1 GiB device copy reads {f_copy:.0f} KiB by FETCH_SIZE and writes "
             f"{w_copy:.0f} KiB by WRITE_SIZE",
             f"fetch_factor: {ff:.5f}", f"write_factor: {wf:.5f}",
             f"launches: {len(f[lm])}",
             f"fetch_bytes_per_launch: {fetch:.0f}", f"write_bytes_per_launch: {write:.0f}",
             f"traffic_bytes_per_launch: {fetch + write:.0f}",
             f"gemm_source_sha256_16: {gemm_source_hash()}"]
    open(out, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        stats(*sys.argv[2:6])
    elif mode == "traffic":
        traffic(*sys.argv[2:6])
    else:
        raise SystemExit(__doc__)
