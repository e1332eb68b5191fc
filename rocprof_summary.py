"""Summarise the rocprofv3 runs of one bench.py workload into profiles/.

python rocprof_summary.py WORKLOAD VARIANT TRACE_DIR FETCH_DIR WRITE_DIR [CLOCK_DIR]
python rocprof_summary.py counters WORKLOAD PASS_DIR [PASS_DIR ...]

The second form writes profiles/counters_<workload>.md from `rocprofv3 --pmc ...` runs of the grouped GEMM
kernels (one directory per counter pass): per kernel the counters averaged over its dispatches and the
derived figures (MFMA busy, VALU busy, LDS busy and bank-conflict stalls, L2 hit rate and read latency,
wavefront wait share).

TRACE_DIR holds the CSV output of `rocprofv3 --kernel-trace --stats -f csv -o run`, FETCH_DIR and WRITE_DIR
that of `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` over a bench.py run that ends with one plain
1 GiB device copy (`--copy-calibration-mib 1024`).  Writes profiles/kernels_<workload>[_<variant>].md
(kernel durations and HBM bytes per dispatch) and records the grouped GEMMs' bytes per launch, scaled by
what the counters read for the known-size copy, in profiles/traffic.json under the fingerprint of the GEMM
code they were taken on (sha256[:16] of csrc/gemm.hip without comments or whitespace; bench.py reports
them only while it matches).  CLOCK_DIR, if given, holds a `--pmc GRBM_COUNT` run: GRBM_COUNT ticks once per
shader clock in each XCD, so per dispatch GRBM_COUNT / duration / XCD count is the average shader clock the
kernel ran at (the chip lowers it below its 2.4 GHz peak under load).
"""
import csv
import glob
import json
import os
import re
import sys
from collections import defaultdict

from sparse_mixture_experts_08_amd.build import code_fingerprint

ROOT = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(ROOT, "sparse_mixture_experts_08_amd", "csrc", "gemm.hip")
COPY_KIB = 1 << 20  # the calibration copy: 1 GiB read and 1 GiB written


def _csv(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    return [r for f in files for r in csv.DictReader(open(f))]


def _counter(d, name):
    """Average value of counter `name` per dispatch, by kernel name; the copy kernel's entry is its largest
    dispatch (the 1 GiB calibration copy; the run's other copies are small input transfers)."""
    vals = defaultdict(list)
    for r in _csv(d, "counter_collection.csv"):
        if r["Counter_Name"] == name:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: ((max(v), 1) if "copyBuffer" in k else (sum(v) / len(v), len(v))) for k, v in vals.items()}


def _clocks(d):
    """Average shader clock (GHz) per dispatch, by kernel name, from a --pmc GRBM_COUNT run."""
    nx = max(int(r.get("Num_Xcc") or 0) for r in _csv(d, "agent_info.csv"))
    vals = defaultdict(list)
    for r in _csv(d, "counter_collection.csv"):
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if r["Counter_Name"] == "GRBM_COUNT" and dur > 0:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]) / dur / nx)
    return nx, {k: (sum(v) / len(v), min(v), max(v), len(v)) for k, v in vals.items()}


def gemm_role(kernel):
    """'up_gemm' / 'down_gemm' for the grouped GEMM kernels, else None."""
    m = re.search(r"grouped_gemm_(w_|f8_)?kernel<([^>]*)>", kernel)
    if not m:
        return None
    args = [a.strip() for a in m.group(2).split(",")]
    up = args[1] if m.group(1) is None else args[0]
    return "up_gemm" if up == "true" else "down_gemm"


# Counter passes of the GEMM profiles (each within one pass's per-block limits: <= 8 SQ, <= 4 TCC, <= 4 TCP).
COUNTER_PASSES = [
    "MfmaUtil VALUBusy LdsUtil LDSBankConflict GRBM_COUNT",
    "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_LDS SQ_INSTS_LDS SQ_INSTS_VALU "
    "SQ_INSTS_MFMA",
    "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_DRAM_sum TCP_PENDING_STALL_CYCLES_sum "
    "TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCP_TOTAL_CACHE_ACCESSES_sum GRBM_GUI_ACTIVE",
    "SQ_LDS_IDX_ACTIVE SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_WAIT_INST_LDS SQ_BUSY_CYCLES SQ_WAVE_CYCLES "
    "SQ_LDS_BANK_CONFLICT TA_BUSY_avr TA_ADDR_STALLED_BY_TC_CYCLES_sum GRBM_GUI_ACTIVE",
    "TA_DATA_STALLED_BY_TC_CYCLES_sum TA_ADDR_STALLED_BY_TD_CYCLES_sum TD_TD_BUSY_sum TD_TC_STALL_sum "
    "TCP_TCP_TA_DATA_STALL_CYCLES_sum TCP_TCR_TCP_STALL_CYCLES_sum TCP_PENDING_STALL_CYCLES_sum GRBM_GUI_ACTIVE "
    "GRBM_COUNT",
]


def counters_main(workload, dirs):
    vals = defaultdict(lambda: defaultdict(list))
    # GRBM_GUI_ACTIVE is read in several passes; keep each pass's own value for the per-pass ratios below
    gui = defaultdict(dict)
    for i, d in enumerate(dirs):
        for r in _csv(d, "counter_collection.csv"):
            if "moe::" in r["Kernel_Name"]:
                vals[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    gui[r["Kernel_Name"]].setdefault(i, []).append(float(r["Counter_Value"]))
    gpu = max((r for d in dirs for r in _csv(d, "agent_info.csv")), key=lambda r: int(r.get("Num_Xcc") or 0))
    nxcc, ncu = int(gpu["Num_Xcc"]), int(gpu["Cu_Count"])
    avg = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}
    lines = [f"# rocprofv3 counters of the grouped GEMMs: {workload}", "",
             "Commands (run from /tmp with TMPDIR=/tmp on an MI355X; R = repository root, OUT = an output "
             "directory; one run per counter pass):", "", "```"]
    bench = f"python3 $R/bench.py --workload {workload} --steps 1 --warmup 1 --no-cpu-baseline --no-peaks"
    for i, p in enumerate(COUNTER_PASSES):
        lines.append(f'rocprofv3 --pmc {p} --kernel-include-regex "grouped_gemm" -f csv -d $OUT/p{i + 1} -o run -- '
                     f"{bench}")
    lines.append(f"python3 $R/rocprof_summary.py counters {workload} " +
                 " ".join(f"$OUT/p{i + 1}" for i in range(len(COUNTER_PASSES))))
    lines += ["```", "", "Derived figures (per dispatch, averaged over dispatches):", "",
              "- MFMA busy, VALU busy, LDS busy, LDS bank-conflict stall: rocprofv3's MfmaUtil, VALUBusy, LdsUtil "
              "and LDSBankConflict (percent of the kernel's active cycles);",
              "- L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS); L2 read latency = TCP_TCC_READ_REQ_LATENCY / "
              "TCP_TCC_READ_REQ (cycles per request, as the L1 sees it);",
              "- wait share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (wavefront cycles waiting on a dependency: "
              "memory, LDS or a barrier); VALU / MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA (SQ_INSTS_VALU "
              "counts the MFMAs too).", "",
              "| kernel | MFMA busy % | VALU busy % | LDS busy % | LDS conflict stall % | L2 hit % | L2 read "
              "latency | wait share % | VALU / MFMA |", "|---|---|---|---|---|---|---|---|---|"]

    def g(c, k):
        return avg[k].get(c)

    def fmt(v, f="{:.1f}"):
        return "–" if v is None else f.format(v)
    for k in sorted(avg, key=lambda k: -(g("GRBM_GUI_ACTIVE", k) or 0)):
        hit, miss = g("TCC_HIT_sum", k), g("TCC_MISS_sum", k)
        lat, req = g("TCP_TCC_READ_REQ_LATENCY_sum", k), g("TCP_TCC_READ_REQ_sum", k)
        wait, wc = g("SQ_WAIT_INST_ANY", k), g("SQ_WAVE_CYCLES", k)
        iv, im = g("SQ_INSTS_VALU", k), g("SQ_INSTS_MFMA", k)
        lines.append(f"| `{k}` | {fmt(g('MfmaUtil', k))} | {fmt(g('VALUBusy', k))} | {fmt(g('LdsUtil', k))} | "
                     f"{fmt(g('LDSBankConflict', k), '{:.2f}')} | "
                     f"{fmt(None if hit is None or miss is None else 100 * hit / max(hit + miss, 1))} | "
                     f"{fmt(None if lat is None or not req else lat / req, '{:.0f}')} | "
                     f"{fmt(None if wait is None or not wc else 100 * wait / wc)} | "
                     f"{fmt(None if iv is None or not im else iv / im, '{:.2f}')} |")
    if len(dirs) >= 5:
        lines += ["", "Vector-memory path (passes 4 and 5; per CU, as a fraction of the kernel's cycles = "
                  f"GRBM_GUI_ACTIVE / {nxcc} XCDs, each pass against its own GRBM_GUI_ACTIVE; {ncu} CUs):", "",
                  "- TD busy = TD_TD_BUSY / CUs; TD stalled by TC = TD_TC_STALL / CUs (the data-return unit waiting "
                  "on the L1 / L2 for the next load's data); TA busy = TA_BUSY_avr; TA stalled by TC = "
                  "TA_ADDR_STALLED_BY_TC_CYCLES / CUs; LDS indexed = SQ_LDS_IDX_ACTIVE / CUs (a sum over the SIMDs "
                  "of each shader engine); LDS wait share = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES.", "",
                  "| kernel | TD busy | TD stalled by TC | TA busy | TA stalled by TC | LDS indexed | "
                  "LDS wait share |", "|---|---|---|---|---|---|---|"]
        for k in sorted(avg, key=lambda k: -(g("GRBM_GUI_ACTIVE", k) or 0)):
            c4 = sum(gui[k].get(3, [0])) / max(len(gui[k].get(3, [])), 1) / nxcc
            c5 = sum(gui[k].get(4, [0])) / max(len(gui[k].get(4, [])), 1) / nxcc
            if not c4 or not c5:
                continue
            td, tds = g("TD_TD_BUSY_sum", k), g("TD_TC_STALL_sum", k)
            ta, tas = g("TA_BUSY_avr", k), g("TA_ADDR_STALLED_BY_TC_CYCLES_sum", k)
            lds, wl, wc = g("SQ_LDS_IDX_ACTIVE", k), g("SQ_WAIT_INST_LDS", k), g("SQ_WAVE_CYCLES", k)
            lines.append(f"| `{k}` | {fmt(None if td is None else td / ncu / c5, '{:.2f}')} | "
                         f"{fmt(None if tds is None else tds / ncu / c5, '{:.2f}')} | "
                         f"{fmt(None if ta is None else ta / c4, '{:.2f}')} | "
                         f"{fmt(None if tas is None else tas / ncu / c4, '{:.2f}')} | "
                         f"{fmt(None if lds is None else lds / ncu / c4, '{:.2f}')} | "
                         f"{fmt(None if wl is None or not wc else wl / wc, '{:.3f}')} |")
    lines += ["", "Raw counter values (average per dispatch):", "", "| kernel | counter | value |", "|---|---|---|"]
    for k in sorted(avg):
        for c in sorted(avg[k]):
            lines.append(f"| `{k}` | {c} | {avg[k][c]:.4g} |")
    lines += ["", "GEMM code fingerprint when measured (sha256[:16] of csrc/gemm.hip without comments or whitespace): "
              f"`{code_fingerprint(GEMM_SRC)}`", ""]
    name = f"counters_{workload}.md"
    open(os.path.join(ROOT, "profiles", name), "w").write("\n".join(lines))
    print(f"wrote profiles/{name}")


def main():
    if sys.argv[1] == "counters":
        counters_main(sys.argv[2], sys.argv[3:])
        return
    workload, variant, trace_dir, fetch_dir, write_dir = sys.argv[1:6]
    clock_dir = sys.argv[6] if len(sys.argv) > 6 else None
    key = workload if variant == "layer" else f"{workload}/{variant}"
    stats = _csv(trace_dir, "kernel_stats.csv")
    fetch, write = _counter(fetch_dir, "FETCH_SIZE"), _counter(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "copyBuffer" in k]
    if not copy or not [k for k in write if "copyBuffer" in k]:
        raise SystemExit("no calibration copy in the counter runs")
    ff = COPY_KIB / fetch[copy[0]][0]
    wf = COPY_KIB / write[[k for k in write if "copyBuffer" in k][0]][0]

    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    moe = [r for r in stats if "moe::" in r["Name"]]
    lines = [f"# rocprofv3 kernel summary: {key}", "",
             "Commands (run from /tmp with TMPDIR=/tmp on an MI355X; R = repository root, OUT = an output "
             "directory):", "", "```"]
    v = f" --variant {variant}"
    bench = f"python3 $R/bench.py --workload {workload}{v}"
    lines.append(f"rocprofv3 --kernel-trace --stats -f csv -d $OUT/trace -o run -- {bench} "
                 "--steps 10 --warmup 2 --no-cpu-baseline --no-peaks")
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        lines.append(f'rocprofv3 --pmc {c} --kernel-include-regex "moe::|copyBuffer" -f csv -d '
                     f"$OUT/{c} -o run -- {bench} --steps 1 --warmup 1 --no-cpu-baseline --no-peaks "
                     "--copy-calibration-mib 1024")
    if clock_dir:
        lines.append(f'rocprofv3 --pmc GRBM_COUNT --kernel-include-regex "moe::" -f csv -d $OUT/GRBM_COUNT -o run '
                     f"-- {bench} --steps 2 --warmup 1 --no-cpu-baseline --no-peaks")
    lines.append(f"python3 $R/rocprof_summary.py {workload} {variant} $OUT/trace $OUT/FETCH_SIZE $OUT/WRITE_SIZE"
                 + (" $OUT/GRBM_COUNT" if clock_dir else ""))
    lines += ["```", "", "## Kernel durations (--kernel-trace --stats; every dispatch in the run, including the "
              "staged pass)", "", "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in moe:
        lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    lines += ["", "## HBM traffic per dispatch (--pmc, averaged over dispatches)", "",
              f"Calibration: one plain device copy of 1 GiB (torch copy_, dispatched as `{copy[0]}`) reads "
              f"FETCH_SIZE = {fetch[copy[0]][0]:.0f} KiB and WRITE_SIZE = "
              f"{write[[k for k in write if 'copyBuffer' in k][0]][0]:.0f} KiB; scale factors FETCH x{ff:.3f}, "
              f"WRITE x{wf:.3f}.", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB (scaled) | written GB (scaled) |",
              "|---|---|---|---|---|---|"]
    rec = {"gemm_code_sha256_16": code_fingerprint(GEMM_SRC),
           "fetch_factor": ff, "write_factor": wf}
    for k in sorted(fetch):
        if "moe::" not in k:
            continue
        fk, n = fetch[k]
        wk = write.get(k, (0.0, 0))[0]
        rb, wb = fk * 1024 * ff / 1e9, wk * 1024 * wf / 1e9
        lines.append(f"| `{k}` | {n} | {fk:.0f} | {wk:.0f} | {rb:.3f} | {wb:.4f} |")
        role = gemm_role(k)
        if role:
            rec[role] = {"kernel": k, "bytes": (rb + wb) * 1e9}
    if clock_dir:
        nx, clk = _clocks(clock_dir)
        lines += ["", "## Average shader clock per dispatch (--pmc GRBM_COUNT / duration / "
                  f"{nx} XCDs; peak 2.4 GHz)", "",
                  "Kernels of a few microseconds read high: the counter window is wider than the kernel.", "",
                  "| kernel | dispatches | average GHz | min GHz | max GHz |", "|---|---|---|---|---|"]
        traced = [r["Name"] for r in moe if r["Name"] in clk]
        order = traced + sorted(k for k in clk if k not in traced)
        for k in order:
            a, lo, hi, n = clk[k]
            lines.append(f"| `{k}` | {n} | {a:.2f} | {lo:.2f} | {hi:.2f} |")
    lines += ["", "GEMM code fingerprint when measured (sha256[:16] of csrc/gemm.hip without comments or whitespace): "
              f"`{rec['gemm_code_sha256_16']}`",
              ""]
    name = f"kernels_{workload}" + ("" if variant == "layer" else f"_{variant}") + ".md"
    open(os.path.join(ROOT, "profiles", name), "w").write("\n".join(lines))
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        traffic = json.load(open(tpath))
    except (OSError, ValueError):
        traffic = {}
    traffic[key] = rec
    json.dump(traffic, open(tpath, "w"), indent=1)
    print(f"wrote profiles/{name}; traffic[{key}]: " +
          ", ".join(f"{r} {rec[r]['bytes'] / 1e9:.2f} GB" for r in ("up_gemm", "down_gemm") if r in rec))


if __name__ == "__main__":
    main()
