"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m speculative_decoding_round_amd.profsum stats  KERNEL_STATS_CSV BENCH_JSON OUT.txt CMD
    python -m speculative_decoding_round_amd.profsum opstats KERNEL_STATS_CSV OPS_JSON OUT.txt CMD
    python -m speculative_decoding_round_amd.profsum traffic FETCH_CSV WRITE_CSV OUT.txt CMD [KERNEL_RE [TITLE]]
    python -m speculative_decoding_round_amd.profsum counter CSV OUT.txt CMD KERNEL_RE COUNTER
    python -m speculative_decoding_round_amd.profsum counters CSV OUT.txt CMD KERNEL_RE TITLE

`stats` lists the kernels of a `rocprofv3 --kernel-trace --stats` run with their average
duration, marks the LM-head GEMM and puts bench.py's own event-timed average beside it.
`opstats` does the same for a `bench.py --only-ops --ops KEY` run (one op's kernels) and puts
the op's event-timed average and roofline fraction beside the profiler's average.
`traffic` reads one `--pmc FETCH_SIZE` and one `--pmc WRITE_SIZE` run (KiB per dispatch),
scales both by what the same counter reads for the plain 1 GiB device copy that
`bench.py --copy-calibration-mb 1024` adds, and records the HBM bytes per launch of the
kernel matching KERNEL_RE (default: the LM head) with a hash of the kernel sources, so
bench.py can tell when they went stale.  `counter` records the per-dispatch average of any
one counter for one kernel (e.g. SQ_INSTS_VALU).
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
# the LM head (role 1): the LDS-ring kernel at one row tile, or the wide kernel (33 .. 160 rows)
LM_HEAD_KERNEL = re.compile(r"k_gemm_ring<1, 8, \d+, false, 1, 1>|k_gemm_wide<\d+, (?:16|32), \d+, false, 1>")


def source_hash(files=("gemm.hip", "common.h")) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def gemm_source_hash() -> str:
    return source_hash(("gemm.hip", "common.h"))


# kernel name pattern -> the sources its code comes from (for staleness of stored counters)
KERNEL_SOURCES = {"k_gemm_ring": ("gemm.hip", "common.h"), "k_gemm_wide": ("gemm.hip", "common.h"),
                  "k_tree_attn_dma": ("attention.hip", "common.h"),
                  "k_lse_merge": ("attention.hip", "common.h"),
                  "k_accept_scan": ("verify.hip", "common.h")}


def sources_for(kernel_re: str):
    for k, v in KERNEL_SOURCES.items():
        if k in kernel_re:
            return v
    return ("gemm.hip", "common.h")


RING_ROLES = {"1": "LM head", "2": "QKV", "3": "O projection", "4": "MLP down", "5": "feature fusion",
              "6": "MLP gate/up (SiLU)"}


def _short(name: str) -> str:
    m = re.search(r"(k_[a-z_0-9]+)(<[^()]*>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else name[:60]


def _role(name: str) -> str:
    m = re.search(r"k_gemm_ring<\d+, \d+, \d+, (?:false|true), (\d+), \d+>", name)
    if m and m.group(1) in RING_ROLES:
        return "  <- " + RING_ROLES[m.group(1)]
    m = re.search(r"k_gemm_wide<\d+, \d+, \d+, (?:false|true), (\d+)>", name)
    if m and m.group(1) in RING_ROLES:
        return "  <- " + RING_ROLES[m.group(1)]
    if re.search(r"k_gemm<[^>]*true>", name):
        return "  <- MLP gate/up (SiLU)"
    return ""


def stats(csv_path, bench_json, out, cmd):
    rows = list(csv.DictReader(open(csv_path)))
    bench = json.loads(open(bench_json).read().strip().splitlines()[-1])
    lines = [f"# rocprofv3 kernel stats, {bench['config']['workload']}", f"command: {cmd}", "",
             f"{'calls':>6} {'avg_us':>10} {'total_%':>8}  kernel"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:24]:
        mark = _role(r["Name"])
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['Percentage']):8.2f}  {_short(r['Name'])}{mark}")
    lm = sorted([r for r in rows if LM_HEAD_KERNEL.search(r["Name"])], key=lambda r: -float(r["TotalDurationNs"]))
    if lm:
        lines += ["", f"LM-head GEMM average (rocprofv3): {float(lm[0]['AverageNs']) / 1e3:.2f} us",
                  f"LM-head GEMM average (bench.py HIP events, same run): "
                  f"{bench['roofline']['avg_launch_us']:.2f} us",
                  f"bench ms_per_step under the profiler: {bench['ms_per_step']}"]
    open(out, "w").write("\n".join(lines) + "\n")


def opstats(csv_path, ops_json, out, cmd):
    rows = list(csv.DictReader(open(csv_path)))
    ops = json.loads(open(ops_json).read().strip().splitlines()[-1])["ops"]
    lines = [f"# rocprofv3 kernel stats, per-op measurement: " + ", ".join(o["op"] + " on " + o["workload"] for o in ops),
             f"command: {cmd}", "", f"{'calls':>6} {'avg_us':>10} {'total_%':>8}  kernel"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"]))[:12]:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['Percentage']):8.2f}  {_short(r['Name'])}")
    lines.append("")
    for o in ops:
        lines.append(f"bench.py (HIP events, same run): {o['op']} on {o['workload']}: {o['avg_launch_us']} us, "
                     f"{o.get('achieved')} {o.get('unit')} = {o.get('frac')} of peak ({o['bound']}-bound)")
    open(out, "w").write("\n".join(lines) + "\n")


def _per_kernel(csv_path):
    agg = defaultdict(list)
    for r in csv.DictReader(open(csv_path)):
        agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def traffic(fetch_csv, write_csv, out, cmd, kernel_re=None, title=None):
    pat = re.compile(kernel_re) if kernel_re else LM_HEAD_KERNEL
    f, w = _per_kernel(fetch_csv), _per_kernel(write_csv)
    copy = [k for k in f if "copyBuffer" in k]
    known = 1 << 20                                     # KiB moved each way by the 1 GiB copy
    f_copy = max(max(f[k]) for k in copy)
    w_copy = max(max(w[k]) for k in copy)
    ff, wf = known / f_copy, known / w_copy
    lm = [k for k in f if pat.search(k)][0]
    fetch = sum(f[lm]) / len(f[lm]) * ff * 1024
    write = sum(w[lm]) / len(w[lm]) * wf * 1024
    lines = [f"# HBM traffic of {title or 'the LM-head GEMM, llama8b workload'} (rocprofv3 --pmc)",
             f"kernel: {_short(lm)}",
             f"command_fetch: {cmd.format(counter='FETCH_SIZE')}",
             f"command_write: {cmd.format(counter='WRITE_SIZE')}",
             f"copy_calibration: 1 GiB device copy reads {f_copy:.0f} KiB by FETCH_SIZE and writes "
             f"{w_copy:.0f} KiB by WRITE_SIZE",
             f"fetch_factor: {ff:.5f}", f"write_factor: {wf:.5f}",
             f"launches: {len(f[lm])}",
             f"fetch_bytes_per_launch: {fetch:.0f}", f"write_bytes_per_launch: {write:.0f}",
             f"traffic_bytes_per_launch: {fetch + write:.0f}",
             f"source_sha256_16: {source_hash(sources_for(_short(lm)))}"]
    open(out, "w").write("\n".join(lines) + "\n")


def counter(csv_path, out, cmd, kernel_re, name):
    pat = re.compile(kernel_re)
    agg = _per_kernel(csv_path)
    k = [k for k in agg if pat.search(k)][0]
    avg = sum(agg[k]) / len(agg[k])
    lines = [f"# {name} per dispatch of {_short(k)} (rocprofv3 --pmc)", f"command: {cmd}",
             f"kernel: {_short(k)}", f"launches: {len(agg[k])}", f"{name.lower()}_per_launch: {avg:.0f}",
             f"source_sha256_16: {source_hash(sources_for(_short(k)))}"]
    open(out, "w").write("\n".join(lines) + "\n")


def counters(csv_path, out, cmd, kernel_re, title, xcds=8, simds=1024):
    """Several counters of one --pmc pass, per dispatch, for every kernel matching KERNEL_RE,
    with the derived rates: MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x cycles,
    GRBM_GUI_ACTIVE summed over the XCDs / XCDs), cycles per MFMA instruction, waiting share of
    wave cycles, and LDS bank-conflict cycles per LDS-active cycle."""
    pat = re.compile(kernel_re)
    agg = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        if pat.search(r["Kernel_Name"]):
            agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = [f"# {title} (rocprofv3 --pmc, per-dispatch averages)", f"command: {cmd}", ""]
    for k, cs in agg.items():
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        n = len(next(iter(cs.values())))
        lines.append(f"kernel: {_short(k)}  ({n} dispatches)")
        lines.append("  " + ", ".join(f"{c} {v:.0f}" for c, v in sorted(avg.items())))
        gui = avg.get("GRBM_GUI_ACTIVE", 0) / xcds
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            lines.append(f"  mfma_busy_fraction: {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (simds * gui):.3f}")
        if avg.get("SQ_INSTS_MFMA"):
            lines.append(f"  cycles_per_mfma: {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / avg['SQ_INSTS_MFMA']:.1f}")
        if avg.get("SQ_WAVE_CYCLES"):
            lines.append(f"  wait_any_share: {avg.get('SQ_WAIT_ANY', 0) / avg['SQ_WAVE_CYCLES']:.3f}, "
                         f"wait_lds_share: {avg.get('SQ_WAIT_INST_LDS', 0) / avg['SQ_WAVE_CYCLES']:.3f}")
        if avg.get("SQ_LDS_IDX_ACTIVE"):
            lines.append(f"  lds_bank_conflict_per_active: {avg.get('SQ_LDS_BANK_CONFLICT', 0) / avg['SQ_LDS_IDX_ACTIVE']:.3f}")
        lines.append(f"  source_sha256_16: {source_hash(sources_for(_short(k)))}")
    open(out, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        stats(*sys.argv[2:6])
    elif mode == "opstats":
        opstats(*sys.argv[2:6])
    elif mode == "traffic":
        traffic(*sys.argv[2:8])
    elif mode == "counter":
        counter(*sys.argv[2:7])
    elif mode == "counters":
        counters(*sys.argv[2:7])
    else:
        raise SystemExit(__doc__)
