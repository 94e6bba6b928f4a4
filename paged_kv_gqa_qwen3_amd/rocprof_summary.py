"""Text summaries of rocprofv3 output for the profiles/ directory.

Two inputs, both CSV directories written by rocprofv3 on the GPU machine:

* a kernel trace (``--kernel-trace --stats``): per-dispatch durations of the
  decode-step kernels, grouped into classes;
* two counter runs (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, one
  counter per run) of a command that also runs one plain 1 GiB device copy
  (bench.py --copy-calibration-mib 1024): the copy's counter values give the
  factor from counter units to bytes, which then scales every kernel's
  counters into HBM bytes per dispatch.

A third summary reads a counter run of the MFMA metrics (``--pmc MfmaUtil
MfmaFlopsBF16 SQ_BUSY_CYCLES``: the share of cycles the matrix cores are busy,
and the bf16 matrix FLOPs per dispatch), with the mean dispatch durations of
a kernel trace of the same workload, into bf16 MFMA TFLOP/s per class.

Usage (repo root):
  python -m paged_kv_gqa_qwen3_amd.rocprof_summary trace <trace_dir> <prefix> <workload> <out.txt> <command...>
  python -m paged_kv_gqa_qwen3_amd.rocprof_summary traffic <fetch_dir> <write_dir> <workload> <kind> <out_prefix>
  python -m paged_kv_gqa_qwen3_amd.rocprof_summary mfma <pmc_dir> <trace_dir> <prefix> <workload> <out.txt> <command...>
"""
from __future__ import annotations

import collections
import csv
import glob
import json
import os
import re
import sys

# Kernel-name substrings -> class (first match wins); GEMV launches are
# classed by their epilogue (the second template argument, any batch width).
CLASSES = (
    ("pf_gemm_kernel<0", "pf_qkv"),
    ("pf_gemm_kernel<1", "pf_o+down"),
    ("pf_gemm_kernel<2", "pf_gate_up"),
    ("pf_attn_kernel", "pf_attention"),
    ("pf_qk_kernel", "pf_qk_rope"),
    ("pf_norm_kernel", "pf_norm"),
    ("pf_embed_kernel", "pf_embed"),
    ("pf_head_rows_kernel", "pf_head_rows"),
    ("stream_step_kernel", "stream_step"),
    ("fused_mlp_kernel", "gate_up+down"),
    ("read_ceiling_kernel", "read_ceiling"),
    ("sample_sum_kernel", "sample_sum"),
    ("sample_nucleus_kernel", "sample_nucleus"),
    ("sample_kernel", "sample"),
    ("attention_kernel", "attention"),
    ("embed_kernel", "embed"),
)
GEMV_MODES = {"4": "qkv", "2": "gate_up", "3": "lm_head", "1": "o_proj+down", "0": "gemv_store"}
# staged items (gemv_kernel<NB, MODE[, RPW]>) and chunk-streamed ones
# (gemv_wide_kernel<NB, MODE, RW>) alike
_GEMV = re.compile(r"gemv_(?:wide_)?kernel<(\d+), (\d+)(?:, \d+)?>")


def kernel_class(name: str):
    for key, cls in CLASSES:
        if key in name:
            return cls
    m = _GEMV.search(name)
    if m:
        return GEMV_MODES.get(m.group(2))
    return None


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def trace_summary(trace_dir: str, prefix: str, workload: str, out_txt: str, command: str) -> None:
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, f"{prefix}_kernel_trace.csv")))))
    dur = collections.defaultdict(list)
    for r in rows:
        c = kernel_class(r["Kernel_Name"])
        if c is not None:
            dur[c].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    stats = list(csv.DictReader(open(_one(os.path.join(trace_dir, f"{prefix}_kernel_stats.csv")))))
    lines = [f"# Kernel durations, workload {workload}", "", "command (repo root, MI355X):",
             "  " + command, "", f'{"class":16s} {"dispatches":>10s} {"mean_us":>10s} {"median_us":>10s}']
    for c in sorted(dur):
        v = sorted(dur[c])
        lines.append(f"{c:16s} {len(v):10d} {sum(v) / len(v):10.2f} {v[len(v) // 2]:10.2f}")
    lines += ["", "rocprofv3 --stats (kernel_stats.csv), top rows:",
              f'{"kernel":64s} {"calls":>6s} {"avg_us":>10s}']
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))[:8]:
        lines.append(f'{r["Name"][:64]:64s} {r["Calls"]:>6s} {float(r["AverageNs"]) / 1e3:10.2f}')
    open(out_txt, "w").write("\n".join(lines) + "\n")


def _counter_rows(run_dir: str, counter: str):
    path = _one(os.path.join(run_dir, "*counter_collection.csv"))
    return [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]


def _calibration(rows) -> float:
    """Counter value of the 1 GiB copy (the copy kernel with the largest grid)."""
    copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
    if not copies:
        raise ValueError("no device copy in the counter run")
    big = max(copies, key=lambda r: int(r["Grid_Size"]))
    return float(big["Counter_Value"])


def traffic_summary(fetch_dir: str, write_dir: str, workload: str, kind: str,
                    out_prefix: str) -> dict:
    """Scaled HBM bytes per dispatch of each kernel class; writes
    <out_prefix>.txt and <out_prefix>.json (with the kernel source sha256 that
    bench.py checks before it reports the figure)."""
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench  # the repo-root benchmark: source hash and algorithmic bytes

    f, w = _counter_rows(fetch_dir, "FETCH_SIZE"), _counter_rows(write_dir, "WRITE_SIZE")
    gib_kib = 1024.0 * 1024.0
    fs, ws = gib_kib / _calibration(f), gib_kib / _calibration(w)

    def per_class(rows):
        d = collections.defaultdict(list)
        for r in rows:
            c = kernel_class(r["Kernel_Name"])
            if c:
                d[c].append(float(r["Counter_Value"]))
        return d

    fc, wc = per_class(f), per_class(w)
    sha = bench.kernel_source_sha256(kind)
    run = (f"python -u bench.py --steps 4 --warmup 1 --reps 1 --no-cpu-baseline --no-prefill "
           f"--no-serve --copy-calibration-mib 1024 --workloads {workload}")
    lines = [f"# HBM traffic per dispatch (rocprofv3 --pmc), workload {workload}", "",
             "commands (repo root, MI355X), one counter per run, then this summary:",
             f"  rocprofv3 --pmc FETCH_SIZE --output-format csv -d {fetch_dir} -o fetch -- {run}",
             f"  rocprofv3 --pmc WRITE_SIZE --output-format csv -d {write_dir} -o write -- {run}",
             f"  python -m paged_kv_gqa_qwen3_amd.rocprof_summary traffic {fetch_dir} {write_dir} "
             f"{workload} {kind} {out_prefix}", "",
             f"kernel source sha256 ({' + '.join(bench.KERNEL_SOURCES[kind])}): {sha}", "",
             f"Calibration: the 1 GiB device copy reads FETCH_SIZE = {_calibration(f):.1f} KiB and "
             f"WRITE_SIZE = {_calibration(w):.1f} KiB",
             f"for 1,048,576 KiB moved each way: FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f}.", "",
             f'{"kernel class":16s} {"dispatches":>10s} {"fetch_KiB":>12s} {"write_KiB":>10s} {"scaled_MB":>10s}']
    traffic = {}
    for c in sorted(fc):
        if c not in wc:
            continue
        fk = sum(fc[c]) / len(fc[c])
        wk = sum(wc[c]) / len(wc[c])
        b = (fk * fs + wk * ws) * 1024.0
        lines.append(f"{c:16s} {len(fc[c]):10d} {fk:12.1f} {wk:10.1f} {b / 1e6:10.2f}")
        traffic[c] = int(round(b))
    rec = {"kernel_source_sha256": sha, "workload": workload, "traffic_bytes_per_launch": traffic,
           "fetch_scale": fs, "write_scale": ws}
    open(out_prefix + ".txt", "w").write("\n".join(lines) + "\n")
    json.dump(rec, open(out_prefix + ".json", "w"), indent=1)
    return rec


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def mfma_summary(pmc_dir: str, trace_dir: str, prefix: str, workload: str, out_txt: str,
                 command: str) -> None:
    """Per kernel class: mean MfmaUtil (% of matrix-core cycles busy over the
    dispatch), bf16 MFMA FLOPs per dispatch and, over the class's mean
    duration in the kernel trace, bf16 MFMA TFLOP/s and its share of the
    2.5 PFLOP/s dense peak."""
    path = _one(os.path.join(pmc_dir, "*counter_collection.csv"))
    rows = list(csv.DictReader(open(path)))
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in rows:
        c = kernel_class(r["Kernel_Name"])
        if c is not None:
            vals[c][r["Counter_Name"]].append(float(r["Counter_Value"]))
    trace = list(csv.DictReader(open(_one(os.path.join(trace_dir, f"{prefix}_kernel_trace.csv")))))
    dur = collections.defaultdict(list)
    for r in trace:
        c = kernel_class(r["Kernel_Name"])
        if c is not None:
            dur[c].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# MFMA activity per dispatch (rocprofv3 --pmc), workload {workload}", "",
             "commands (repo root, MI355X):", "  " + command, "",
             "MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), in %;",
             "MfmaFlopsBF16 = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (one 16x16x32 bf16 MFMA = 16384);",
             "TFLOP/s = MfmaFlopsBF16 / mean duration of the class in the kernel trace.", "",
             f'{"class":16s} {"dispatches":>10s} {"MfmaUtil_%":>10s} {"GFLOP":>10s} '
             f'{"mean_us":>9s} {"TFLOP/s":>9s} {"of_peak":>8s} {"SQ_BUSY_Mcyc":>12s}']
    for c in sorted(vals):
        v = vals[c]
        util = v.get("MfmaUtil", [])
        fl = v.get("MfmaFlopsBF16", [])
        busy = v.get("SQ_BUSY_CYCLES", [])
        if not fl:
            continue
        mf = sum(fl) / len(fl)
        mu = sum(util) / len(util) if util else float("nan")
        sb = sum(busy) / len(busy) / 1e6 if busy else float("nan")
        d = sum(dur[c]) / len(dur[c]) if dur.get(c) else float("nan")
        tf = mf / (d * 1e-6) / 1e12 if dur.get(c) else float("nan")
        lines.append(f"{c:16s} {len(fl):10d} {mu:10.2f} {mf / 1e9:10.2f} {d:9.2f} {tf:9.2f} "
                     f"{tf / MFMA_BF16_PEAK_TFLOPS:8.4f} {sb:12.2f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")


def main(argv):
    if len(argv) >= 6 and argv[1] == "trace":
        trace_summary(argv[2], argv[3], argv[4], argv[5], " ".join(argv[6:]))
    elif len(argv) == 7 and argv[1] == "traffic":
        print(json.dumps(traffic_summary(argv[2], argv[3], argv[4], argv[5], argv[6]), indent=1))
    elif len(argv) >= 7 and argv[1] == "mfma":
        mfma_summary(argv[2], argv[3], argv[4], argv[5], argv[6], " ".join(argv[7:]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
