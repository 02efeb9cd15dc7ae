"""Turn rocprofv3 output into the short text summaries kept under profiles/.

    python -m io_aware_exact_09_amd.profiles stats <kernel_stats.csv> <out.md> "<command>" \
        [<kernel_trace.csv> <warmup> <steps> [<secondary steps before the headline>]]
    python -m io_aware_exact_09_amd.profiles traffic <fetch_dir> <write_dir> <workload> \
        <out.json> "<fetch command>" "<write command>"
    python -m io_aware_exact_09_amd.profiles counters <out.md> <workload> \
        <pass_dir>=<command> ...

``counters`` reads ``--pmc`` passes of the same bench command and tabulates,
per kernel, the counters and the ratios derived from them (formulas in the
output).  ``stats`` condenses a ``--kernel-trace --stats`` run (per-kernel calls and
average duration).  ``traffic`` reads two ``--pmc FETCH_SIZE`` /
``--pmc WRITE_SIZE`` runs of ``bench.py --copy-probe``: the probe is a plain
device-to-device copy of a known number of bytes, and the ratio of those bytes
to what the counter reports for it calibrates the counter for the attention
kernels of the same run.  The JSON records, per attention kernel, the
calibrated HBM bytes per launch and a hash of the kernel sources, so that
bench.py reports the traffic only while the kernels are unchanged.
"""

from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")

KERNELS = ("fa_fwd_kernel", "fa_fwd_pp_kernel", "fa_fwd_combine_kernel", "fa_bwd_delta_kernel",
           "fa_bwd_dkdv_kernel", "fa_bwd_dkdv_reduce_kernel", "fa_bwd_dq_kernel",
           "fa_bwd_dq_reduce_kernel", "fa_decode_split_kernel", "fa_decode_combine_kernel",
           "fa_fwd_fp8_kernel")

# Device sources of each kernel family (host-side files such as fa_api.cpp
# do not change what a kernel does on the GPU).
SOURCES = {
    "train": ("fa_common.hpp", "fa_launch.hpp", "fa_rows.hpp", "fa_fwd.hip", "fa_bwd.hip"),
    "decode": ("fa_common.hpp", "fa_decode.hpp", "fa_decode.hip"),
    "fp8": ("fa_common.hpp", "fa_launch.hpp", "fa_fwd_fp8.hip"),
}


def family(workload: str) -> str:
    if workload.startswith("decode"):
        return "decode"
    return "fp8" if workload.endswith("fp8") else "train"


def source_hash(fam: str = "train") -> str:
    """Hash of the device sources the kernels of family `fam` are built from."""
    h = hashlib.sha256()
    for name in SOURCES[fam]:
        with open(os.path.join(HERE, "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


PROBE = "probe:neg"      # bench.py --copy-probe runs one torch.neg over a known size


def short_name(kernel_name: str) -> str:
    for k in KERNELS:
        if k in kernel_name:
            return k
    if "neg_kernel" in kernel_name:
        return PROBE
    if "reduce_kernel" in kernel_name:
        return "reduction (cache eviction):" + kernel_name[:40]
    if "FillFunctor" in kernel_name or "fill" in kernel_name.lower():
        return "fill:" + kernel_name[:40]
    if "copy" in kernel_name.lower() or "elementwise" in kernel_name:
        return "copy:" + kernel_name[:60]
    return kernel_name[:60]


def _rows(path_or_dir: str, suffix: str):
    paths = [path_or_dir] if path_or_dir.endswith(".csv") else \
        glob.glob(os.path.join(path_or_dir, "**", f"*{suffix}"), recursive=True)
    for p in paths:
        with open(p) as f:
            yield from csv.DictReader(f)


def stats_summary(stats_csv: str, command: str, trace_csv: str | None = None,
                  warmup: int = 0, steps: int = 0, skip: int = 0) -> str:
    """Per-kernel calls and durations from a --kernel-trace --stats run.

    With the per-dispatch trace and the bench's step counts (one launch of
    each kernel per step), a last column averages only the dispatches of the
    headline's timed steps, the launches the bench's HIP events time: the
    `steps` launches that follow the first `warmup + skip` ones (warm-up
    steps, then the bench's secondary steps).
    """
    timed = {}
    if trace_csv:
        per = {}
        rows = sorted(_rows(trace_csv, "kernel_trace.csv"), key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            per.setdefault(short_name(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        for k, v in per.items():
            if len(v) >= warmup + skip + steps and steps > 0:
                timed[k] = statistics.fmean(v[warmup + skip:warmup + skip + steps])
    lines = ["# rocprofv3 kernel-trace summary", "", f"Command: `{command}`", ""]
    head = "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |"
    if timed:
        a, b = warmup + skip + 1, warmup + skip + steps
        lines += [f"Last column: average over dispatches {a}..{b} of each kernel: the {steps} "
                  f"headline steps, after {warmup} warm-up steps and {skip} secondary steps (the "
                  "launches the bench's HIP events average for its headline and roofline; each "
                  "follows a cache-evicting read of a device buffer, the reduction kernel listed "
                  "separately). "
                  "The other columns count every dispatch.", ""]
        head += " timed steps average (us) |"
    lines += [head, "|" + "---|" * (head.count("|") - 1)]
    for r in _rows(stats_csv, "kernel_stats.csv"):
        k = short_name(r["Name"])
        line = "| {} | {} | {:.1f} | {:.1f} | {:.1f} | {:.1f}% |".format(
            k, r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"]))
        if timed:
            line += f" {timed[k]:.1f} |" if k in timed else " |"
        lines.append(line)
    return "\n".join(lines) + "\n"


def _counter_per_kernel(d: str, counter: str):
    vals = {}
    for r in _rows(d, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return vals


def traffic(fetch_dir: str, write_dir: str, copy_bytes: int) -> dict:
    """Calibrated HBM bytes per launch of each attention kernel."""
    out = {}
    for counter, d, key in (("FETCH_SIZE", fetch_dir, "read"), ("WRITE_SIZE", write_dir, "write")):
        per = _counter_per_kernel(d, counter)
        copies = per.get(PROBE, [])
        probe = max(copies) if copies else None
        factor = copy_bytes / (probe * 1024.0) if probe else None
        out[f"{key}_calibration"] = {"probe_bytes": copy_bytes,
                                     "counter_kib": probe, "factor": factor}
        for k in KERNELS:
            if k in per and factor:
                out.setdefault(k, {})[f"{key}_bytes"] = statistics.median(per[k]) * 1024.0 * factor
                out[k][f"{key}_counter_kib"] = statistics.median(per[k])
    return out


# Hardware constants of the MI355X used to normalise counters.
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def counters_table(passes, workload: str) -> str:
    """Per-kernel counter averages over dispatches, merged over passes."""
    vals = {}
    for d, _ in passes:
        for r in _rows(d, "counter_collection.csv"):
            k = short_name(r["Kernel_Name"])
            if k not in KERNELS:
                continue
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    avg = {k: {c: statistics.mean(v) for c, v in cs.items()} for k, cs in vals.items()}

    def ratio(k, f):
        try:
            return f(avg[k])
        except (KeyError, ZeroDivisionError):
            return None

    derived = [
        ("clock cycles per dispatch", "GRBM_GUI_ACTIVE / 8 (summed over the 8 XCDs)",
         lambda c: c["GRBM_GUI_ACTIVE"] / N_XCD),
        ("MFMA busy", "SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)",
         lambda c: c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / N_XCD * N_SIMD)),
        ("MFMA busy cycles per MFMA", "SQ_VALU_MFMA_BUSY_CYCLES / SQ_INSTS_MFMA",
         lambda c: c["SQ_VALU_MFMA_BUSY_CYCLES"] / c["SQ_INSTS_MFMA"]),
        ("VALU per MFMA", "(SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA",
         lambda c: (c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]) / c["SQ_INSTS_MFMA"]),
        ("exp per MFMA", "SQ_INSTS_VALU_TRANS_F32 / SQ_INSTS_MFMA",
         lambda c: c["SQ_INSTS_VALU_TRANS_F32"] / c["SQ_INSTS_MFMA"]),
        ("LDS per MFMA", "SQ_INSTS_LDS / SQ_INSTS_MFMA",
         lambda c: c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"]),
        ("MFMA/VALU co-issue", "SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES",
         lambda c: c["SQ_VALU_MFMA_COEXEC_CYCLES"] / c["SQ_VALU_MFMA_BUSY_CYCLES"]),
        ("LDS bank conflicts per access", "SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT)",
         lambda c: c["SQ_LDS_BANK_CONFLICT"] / (c["SQ_LDS_IDX_ACTIVE"] - c["SQ_LDS_BANK_CONFLICT"])),
        ("LDS busy", "SQ_LDS_IDX_ACTIVE / (cycles x 256 CUs)",
         lambda c: c["SQ_LDS_IDX_ACTIVE"] / (c["GRBM_GUI_ACTIVE"] / N_XCD * N_CU)),
        ("wave time waiting (any)", "SQ_WAIT_ANY / SQ_WAVE_CYCLES",
         lambda c: c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]),
        ("wave time waiting to issue", "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
         lambda c: c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]),
        ("wave time waiting to issue LDS", "SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES",
         lambda c: c["SQ_WAIT_INST_LDS"] / c["SQ_WAVE_CYCLES"]),
        ("wave time issuing", "SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES",
         lambda c: c["SQ_ACTIVE_INST_ANY"] / c["SQ_WAVE_CYCLES"]),
        ("VALU issue time per SIMD", "4 SQ_ACTIVE_INST_VALU / (cycles x 1024 SIMDs)",
         lambda c: 4 * c["SQ_ACTIVE_INST_VALU"] / (c["GRBM_GUI_ACTIVE"] / N_XCD * N_SIMD)),
        ("LDS issue time per SIMD", "4 SQ_ACTIVE_INST_LDS / (cycles x 1024 SIMDs)",
         lambda c: 4 * c["SQ_ACTIVE_INST_LDS"] / (c["GRBM_GUI_ACTIVE"] / N_XCD * N_SIMD)),
        ("integer VALU per MFMA", "SQ_INSTS_VALU_INT32 / SQ_INSTS_MFMA",
         lambda c: c["SQ_INSTS_VALU_INT32"] / c["SQ_INSTS_MFMA"]),
        ("convert VALU per MFMA", "SQ_INSTS_VALU_CVT / SQ_INSTS_MFMA",
         lambda c: c["SQ_INSTS_VALU_CVT"] / c["SQ_INSTS_MFMA"]),
        ("fp32 FMA per MFMA", "SQ_INSTS_VALU_FMA_F32 / SQ_INSTS_MFMA",
         lambda c: c["SQ_INSTS_VALU_FMA_F32"] / c["SQ_INSTS_MFMA"]),
        ("scalar ALU per MFMA", "SQ_INSTS_SALU / SQ_INSTS_MFMA",
         lambda c: c["SQ_INSTS_SALU"] / c["SQ_INSTS_MFMA"]),
        ("L2 hit rate", "TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)",
         lambda c: c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])),
    ]
    ks = [k for k in KERNELS if k in avg]
    lines = [f"# rocprofv3 counters, workload `{workload}`", "",
             "Averages over the profiled dispatches; SQ counters are summed over the chip by "
             "rocprofv3, GRBM_GUI_ACTIVE over the 8 XCDs.", "",
             "Commands (one `--pmc` pass each):", ""]
    lines += [f"* `{cmd}`" for _, cmd in passes]
    lines += ["", "| derived | formula | " + " | ".join(ks) + " |",
              "|---|---|" + "---|" * len(ks)]
    for name, formula, f in derived:
        cells = []
        for k in ks:
            v = ratio(k, f)
            cells.append("" if v is None else (f"{v:.0f}" if v > 100 else f"{v:.3f}"))
        lines.append(f"| {name} | {formula} | " + " | ".join(cells) + " |")
    lines += ["", "| counter | " + " | ".join(ks) + " |", "|---|" + "---|" * len(ks)]
    for c in sorted({c for k in ks for c in avg[k]}):
        lines.append(f"| {c} | " + " | ".join(f"{avg[k][c]:.4g}" if c in avg[k] else "" for k in ks) + " |")
    return "\n".join(lines) + "\n"


def main(argv):
    if argv[0] == "stats":
        extra = (argv[4], int(argv[5]), int(argv[6])) if len(argv) > 6 else ()
        if len(argv) > 7:
            extra += (int(argv[7]),)
        text = stats_summary(argv[1], argv[3], *extra)
        open(argv[2], "w").write(text)
        print(text)
    elif argv[0] == "traffic":
        fetch_dir, write_dir, workload, out_path, cmd_f, cmd_w = argv[1:7]
        copy_bytes = int(os.environ.get("FA_COPY_PROBE_BYTES", 512 << 20))
        t = traffic(fetch_dir, write_dir, copy_bytes)
        t.update({"workload": workload, "source_hash": source_hash(family(workload)),
                  "commands": {"FETCH_SIZE": cmd_f, "WRITE_SIZE": cmd_w}})
        json.dump(t, open(out_path, "w"), indent=1)
        print(json.dumps(t, indent=1))
    elif argv[0] == "counters":
        out_path, workload = argv[1], argv[2]
        passes = [tuple(a.split("=", 1)) for a in argv[3:]]
        text = counters_table(passes, workload)
        open(out_path, "w").write(text)
        print(text)
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
