"""Summaries of rocprofv3 output for the profiles/ folder (host-side text
processing only; nothing here touches a GPU).

    python -m xlstm_mlstm_matrix_amd.rocprof_summary stats  STATS_CSV TRACE_CSV OUT_MD "COMMAND" [TAIL]
    python -m xlstm_mlstm_matrix_amd.rocprof_summary traffic NAME KERNEL_REGEX \
        FETCH_CSV WRITE_CSV OUT_DIR "FETCH_COMMAND" "WRITE_COMMAND"
    python -m xlstm_mlstm_matrix_amd.rocprof_summary sq KERNEL_REGEX COUNTER_CSV OUT_MD "COMMAND"

`stats` turns the kernel statistics of `rocprofv3 --kernel-trace --stats
-f csv` into a markdown table, followed by the same durations split into runs
of consecutive dispatches of one kernel (one benchmark line launches a kernel
many times in a row; the same kernel in another line forms another run),
with the average of each run's last TAIL dispatches (default 100, the
benchmark's timed steps; its untimed warmup steps come first).  `sq` turns a
counter-collection CSV of SQ/GRBM counters into a table of medians per
dispatch with derived utilisations.  `traffic` reads two counter-collection CSVs
(`rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE`, KiB per dispatch) of a
run that also executed the benchmark's 1 GiB streaming probe (`torch.neg`
over 2^28 float32: 1 GiB read, 1 GiB written).  The probe's counter readings
give the factor from counter units to bytes; the kernel's median reading
per dispatch times that factor is its HBM traffic per launch.  The result
goes to OUT_DIR/NAME_traffic.json (read by bench.py when the kernel sources
still hash to the recorded value) and OUT_DIR/NAME_traffic.md.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join("xlstm_mlstm_matrix_amd", "csrc")
PROBE_REGEX = r"neg"
PROBE_BYTES = 1 << 30


# the device-code files each measured line's kernels are compiled from (a
# change to any of them invalidates that line's measured traffic)
KERNEL_FILES = {
    "prefill_7b": ["common.hpp", "prefill.hip", "prefill_ws.hpp", "prefill_bf16.hpp",
                   "prefill_kernel.hpp"],
    "decode": ["common.hpp", "step.hip"],
    "backward_7b": ["common.hpp", "backward.hip"],
}


def kernel_sources(name=None):
    if name is not None:
        return [os.path.join(CSRC, f) for f in KERNEL_FILES[name]]
    return sorted(os.path.join(CSRC, f) for f in os.listdir(os.path.join(ROOT, CSRC))
                  if f.endswith((".hip", ".hpp", ".cpp")))


def src_hash(name=None) -> str:
    """Hash of the kernel source files of one measured line (all of them when
    name is None)."""
    h = hashlib.sha256()
    for p in kernel_sources(name):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_counter(path: str, counter: str):
    """{dispatch id: (kernel name, value)} for one counter."""
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            d = int(row["Dispatch_Id"])
            name, val = row["Kernel_Name"], float(row["Counter_Value"])
            if d in out:  # several rows for one dispatch (per-instance): sum them
                val += out[d][1]
            out[d] = (name, val)
    return out


def median_for(readings, regex: str):
    """Median reading per dispatch of the kernels matching regex; when several
    kernels match (a step made of more than one launch, each launched once per
    step) the sum of each kernel's median: the reading per step."""
    by_name = {}
    for (n, v) in readings.values():
        if re.search(regex, n):
            by_name.setdefault(n, []).append(v)
    if not by_name:
        raise SystemExit(f"no dispatch matches {regex!r}")
    return (sum(statistics.median(v) for v in by_name.values()),
            min(len(v) for v in by_name.values()))


def kernel_runs(trace_csv: str, min_len: int = 3, span: int = 2):
    """Runs of dispatches of one kernel: (name, first dispatch id, durations
    in ns).  A run goes on while the kernel's next dispatch comes at most
    `span` dispatches later, so a kernel that alternates with another one (a
    step of two launches) still forms one run."""
    with open(trace_csv, newline="") as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    runs, open_run = [], {}
    for i, r in enumerate(rows):
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        name = r["Kernel_Name"]
        if name in open_run and i - open_run[name][0] <= span:
            open_run[name][1][2].append(d)
            open_run[name][0] = i
        else:
            run = (name, int(r["Dispatch_Id"]), [d])
            runs.append(run)
            open_run[name] = [i, run]
    return [x for x in runs if len(x[2]) >= min_len]


def stats(stats_csv: str, trace_csv: str, out_md: str, command: str, tail: int = 100) -> None:
    with open(stats_csv, newline="") as f:
        rows = list(csv.DictReader(f))
    lines = ["# Kernel trace statistics", "", "Command (repository root, one MI355X):", "",
             "```", command, "```", "",
             "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Total (ms) | % |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    lines += ["", "Runs of at least 3 consecutive dispatches of one kernel (in launch order):", "",
              f"| Kernel | First dispatch | Calls | Average (us) | Average of last {tail} (us) | Median (us) "
              "| Min (us) | Max (us) |",
              "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for name, first, ds in kernel_runs(trace_csv):
        last = ds[-tail:]
        lines.append(f"| `{name}` | {first} | {len(ds)} | {statistics.mean(ds) / 1e3:.2f} | "
                     f"{statistics.mean(last) / 1e3:.2f} | "
                     f"{statistics.median(ds) / 1e3:.2f} | {min(ds) / 1e3:.2f} | {max(ds) / 1e3:.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def traffic(name: str, kernel_regex: str, fetch_csv: str, write_csv: str, out_dir: str,
            fetch_cmd: str, write_cmd: str) -> dict:
    fr = read_counter(fetch_csv, "FETCH_SIZE")
    wr = read_counter(write_csv, "WRITE_SIZE")
    kf, nkf = median_for(fr, kernel_regex)
    kw, nkw = median_for(wr, kernel_regex)
    pf, npf = median_for(fr, PROBE_REGEX)
    pw, npw = median_for(wr, PROBE_REGEX)
    sf, sw = PROBE_BYTES / pf, PROBE_BYTES / pw  # bytes per counter unit
    rec = {
        "kernel_regex": kernel_regex, "kernel_src_sha": src_hash(name),
        "kernel_files": KERNEL_FILES[name],
        "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
        "dispatches": [nkf, nkw],
        "probe": {"kernel_regex": PROBE_REGEX, "bytes_read": PROBE_BYTES, "bytes_written": PROBE_BYTES,
                  "fetch_reading": pf, "write_reading": pw, "dispatches": [npf, npw]},
        "bytes_per_unit": {"fetch": sf, "write": sw},
        "bytes_read_per_launch": kf * sf, "bytes_written_per_launch": kw * sw,
        "bytes_per_launch": kf * sf + kw * sw,
        "commands": {"fetch": fetch_cmd, "write": write_cmd},
    }
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{name}_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    md = [f"# HBM traffic of `{kernel_regex}` ({name}, per step: the sum over the matching kernels)", "",
          "Counter passes (repository root, one MI355X), one counter each:", "",
          "```", fetch_cmd, write_cmd, "```", "",
          f"- FETCH_SIZE median per dispatch: {kf:.0f} ({nkf} dispatches)",
          f"- WRITE_SIZE median per dispatch: {kw:.0f} ({nkw} dispatches)",
          f"- probe (`{PROBE_REGEX}`, 1 GiB read + 1 GiB written): FETCH_SIZE {pf:.0f}, "
          f"WRITE_SIZE {pw:.0f} -> {sf:.1f} and {sw:.1f} bytes per counter unit",
          f"- traffic per launch: read {kf * sf / 1e6:.1f} MB, written {kw * sw / 1e6:.1f} MB, "
          f"total {(kf * sf + kw * sw) / 1e6:.1f} MB",
          f"- kernel sources hash: {rec['kernel_src_sha']}", ""]
    with open(os.path.join(out_dir, f"{name}_traffic.md"), "w") as f:
        f.write("\n".join(md))
    return rec


SQ_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
               "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS"]
N_SIMD, N_XCD = 256 * 4, 8  # MI355X: 256 compute units of 4 SIMDs, in 8 XCDs


def sq(kernel_regex: str, counter_csv: str, out_md: str, command: str) -> None:
    vals = {}
    with open(counter_csv, newline="") as f:
        for row in csv.DictReader(f):
            if re.search(kernel_regex, row["Kernel_Name"]):
                key = (row["Counter_Name"], int(row["Dispatch_Id"]))
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    per = {}
    for (name, _), v in vals.items():
        per.setdefault(name, []).append(v)
    m = {k: statistics.median(v) for k, v in per.items()}
    n = len(per.get("GRBM_GUI_ACTIVE", []))
    lines = [f"# SQ counters of `{kernel_regex}`", "", "Command (repository root, one MI355X):", "",
             "```", command, "```", "", f"Median over {n} dispatches (each value summed over the whole GPU):", "",
             "| Counter | Value |", "|---|---:|"]
    lines += [f"| {k} | {m[k]:.0f} |" for k in SQ_COUNTERS if k in m]
    if all(k in m for k in SQ_COUNTERS):
        cyc = m["GRBM_GUI_ACTIVE"] / N_XCD
        other = m["SQ_INSTS_VALU"] - m["SQ_INSTS_MFMA"]
        lines += ["", f"Derived ({N_SIMD // 4} compute units x 4 SIMDs, {N_XCD} XCDs):", "",
                  f"- kernel length: GRBM_GUI_ACTIVE / {N_XCD} = {cyc:.0f} cycles",
                  f"- MFMA busy per SIMD: SQ_VALU_MFMA_BUSY_CYCLES / {N_SIMD} / kernel cycles = "
                  f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / N_SIMD / cyc * 100:.1f}%",
                  f"- MFMA instructions: {m['SQ_INSTS_MFMA']:.0f} "
                  f"({m['SQ_VALU_MFMA_BUSY_CYCLES'] / m['SQ_INSTS_MFMA']:.1f} busy cycles each)",
                  f"- non-MFMA VALU instructions: {other:.0f} = {other / m['SQ_INSTS_MFMA']:.1f} per MFMA; at 4 "
                  f"cycles per wave64 instruction {other * 4 / N_SIMD / cyc * 100:.1f}% of each SIMD's cycles",
                  f"- LDS instructions: {m['SQ_INSTS_LDS']:.0f}", ""]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv):
    if len(argv) >= 1 and argv[0] == "stats" and len(argv) in (5, 6):
        stats(argv[1], argv[2], argv[3], argv[4], *(int(x) for x in argv[5:]))
    elif len(argv) >= 1 and argv[0] == "sq" and len(argv) == 5:
        sq(argv[1], argv[2], argv[3], argv[4])
    elif len(argv) >= 1 and argv[0] == "traffic" and len(argv) == 8:
        rec = traffic(*argv[1:])
        print(json.dumps({k: rec[k] for k in ("bytes_read_per_launch", "bytes_written_per_launch",
                                              "bytes_per_launch")}))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
