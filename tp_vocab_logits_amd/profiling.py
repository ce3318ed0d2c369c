"""Turn rocprofv3 CSV output into the short summaries kept under ``profiles/``.

Two reports:

``kernels``  -- per-kernel call counts and durations from a
    ``--kernel-trace --stats -f csv`` run (``*_kernel_stats.csv``), with the
    algorithmic bandwidth of the gather kernels (5 * M * V * 2 bytes per call).

``counters`` -- HBM-side traffic of the fused gather from two ``--pmc`` runs
    (``FETCH_SIZE`` then ``WRITE_SIZE``, KiB per dispatch) over
    ``bench.py --pmc-probe``. Each counter is scaled by what it reads for the
    plain 256 MiB copy in the same run (``__amd_rocclr_copyBuffer``), so the
    traffic is in bytes per launch. The summary records a hash of the sources
    that fix the gather kernels and their launch shapes; ``bench.py`` reports
    the traffic only while that hash still matches.

Usage::

    python -m tp_vocab_logits_amd.profiling kernels STATS_CSV --command CMD --out FILE.md [--trace TRACE_CSV]
    python -m tp_vocab_logits_amd.profiling counters FETCH_CSV WRITE_CSV \\
        --command-fetch CMD --command-write CMD --out FILE.json
    python -m tp_vocab_logits_amd.profiling sq CSV [CSV ...] --kernel NAME \\
        --command CMD [--command CMD ...] --out FILE.md
    python -m tp_vocab_logits_amd.profiling clock CSV --kernel NAME --command CMD --out FILE.md

``sq`` -- median SQ/TCC/GRBM counters of a kernel over several ``--pmc`` runs,
    with the shader clock, MFMA busy fraction and waits derived from them.

``clock`` -- one ``--pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES`` run over
    many back-to-back dispatches of a kernel: each dispatch's duration, shader
    clock and MFMA busy fraction, in launch order.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
# the sources that fix the gather kernels and their launch shapes
KERNEL_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("hg_kernels.hip", "hg_internal.h", "hg_api.cpp")]
COPY_BYTES = 256 << 20                    # the plain copy of bench.py --pmc-probe
M256_BYTES = 5 * 256 * 163840 * 2        # algorithmic bytes of one M=256 gather


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0] if not name.startswith("void ") else name[5:].split("(")[0]


def _dispatches(trace_csv: str | None) -> list[tuple[str, int, float]]:
    """(kernel name, grid threads, duration ns) of every dispatch in a
    ``*_kernel_trace.csv``."""
    if not trace_csv:
        return []
    out = []
    for r in csv.DictReader(open(trace_csv)):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        out.append((r["Kernel_Name"], grid, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def _stats(ns: list[float]) -> str:
    return (f"{len(ns)} | {statistics.mean(ns) / 1e3:.3f} | {statistics.median(ns) / 1e3:.3f} | "
            f"{min(ns) / 1e3:.3f} | {max(ns) / 1e3:.3f}")


def m1_fused_times(trace_csv: str) -> dict | None:
    """Median duration of the M=1 decode fused gather in a kernel trace: the
    most frequent fused launch shape (the timed loop of bench.py)."""
    groups: dict[tuple[str, int], list[float]] = {}
    for name, grid, ns in _dispatches(trace_csv):
        n = short_name(name)
        if n.startswith("hg::k_fused<"):
            groups.setdefault((n, grid), []).append(ns)
    if not groups:
        return None
    key = max(groups, key=lambda k: len(groups[k]))
    ns = groups[key]
    return {"kernel": key[0], "grid_threads": key[1], "calls": len(ns),
            "median_us": round(statistics.median(ns) / 1e3, 3),
            "mean_us": round(statistics.mean(ns) / 1e3, 3),
            "min_us": round(min(ns) / 1e3, 3),
            "kernel_source_sha256_16": kernel_source_hash()}


def m1_split_times(trace_csv: str, grid_threads: int) -> dict | None:
    """Medians of the split variant's two launches (``k_push``, ``k_collect``)
    at the M=1 fused gather's grid, and their sum: the split M=1 gather's
    kernel time."""
    groups: dict[str, dict[str, list[float]]] = {"push": {}, "collect": {}}
    for name, grid, ns in _dispatches(trace_csv):
        n = short_name(name)
        for part, prefix in (("push", "hg::k_push<"), ("collect", "hg::k_collect<")):
            if n.startswith(prefix) and grid == grid_threads:
                groups[part].setdefault(n, []).append(ns)
    out: dict = {}
    for part, g in groups.items():
        if not g:
            return None
        k = max(g, key=lambda n: len(g[n]))
        out[part] = {"kernel": k, "calls": len(g[k]),
                     "median_us": round(statistics.median(g[k]) / 1e3, 3)}
    out["sum_median_us"] = round(out["push"]["median_us"] + out["collect"]["median_us"], 3)
    return out


def kernels_report(stats_csv: str, command: str, trace_csv: str | None = None) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    disp = _dispatches(trace_csv)
    lines = ["# rocprofv3 kernel summary", "", "Command (TMPDIR=/tmp; paths relative to the repository root):", "",
             "    " + command, "",
             "Per kernel name (the `--stats` table):", "",
             "| kernel | calls | avg us | min us | max us | share |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.3f} | "
                     f"{float(r['MinNs'])/1e3:.3f} | {float(r['MaxNs'])/1e3:.3f} | "
                     f"{float(r['Percentage']):.1f} % |")
    lines += ["", f"Kernel source hash: `{kernel_source_hash()}`", ""]
    if not disp:
        return "\n".join(lines) + "\n"
    # One instantiation serves several row counts, so the per-name figures mix
    # workloads; the trace separates them by launch shape (grid) and, where
    # two row counts share a grid, by duration.
    groups: dict[tuple[str, int], list[float]] = {}
    for name, grid, ns in disp:
        groups.setdefault((short_name(name), grid), []).append(ns)
    lines += ["Per kernel and grid (from the kernel trace):", "",
              "| kernel | grid threads | calls | avg us | median us | min us | max us |",
              "|---|---|---|---|---|---|---|"]
    for (n, grid), ns in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{n}` | {grid} | {_stats(ns)} |")
    lines.append("")
    fused = [(n, g, ns) for (n, g), v in groups.items() if n.startswith("hg::k_fused<") for ns in v]
    # M=256 (about 60 us) is the only fused gather of the run above 40 us.
    big = [ns for _, _, ns in fused if ns > 40e3]
    if big:
        avg = statistics.mean(big) * 1e-9
        lines.append(f"M=256 fused gather (k_fused dispatches above 40 us): {len(big)} calls, "
                     f"{avg * 1e6:.2f} us average, {statistics.median(big) / 1e3:.2f} us median -> "
                     f"{M256_BYTES / avg / 1e9:.1f} GB/s algorithmic ({M256_BYTES / avg / 8e12 * 100:.1f} % of 8 TB/s).")
    # M=1 decode: the most frequent fused launch shape (the timed loop).
    if fused:
        counts: dict[tuple[str, int], int] = {}
        for n, g, _ in fused:
            counts[(n, g)] = counts.get((n, g), 0) + 1
        key = max(counts, key=counts.get)
        ns = groups[key]
        lines.append(f"M=1 decode fused gather (`{key[0]}`, grid {key[1]} threads, the most frequent fused "
                     f"launch): {len(ns)} calls, {statistics.mean(ns) / 1e3:.3f} us average, "
                     f"{statistics.median(ns) / 1e3:.3f} us median, {min(ns) / 1e3:.3f} us minimum.")
    return "\n".join(lines) + "\n"


def _per_kernel(csv_path: str, counter: str) -> dict[str, list[float]]:
    out: dict[str, list[float]] = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def counters_report(fetch_csv: str, write_csv: str, cmd_fetch: str, cmd_write: str) -> dict:
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    copy = next(k for k in fetch if "copyBuffer" in k)
    fused = next(k for k in fetch if "k_fused" in k)
    copy_kib = COPY_BYTES / 1024
    f_factor = copy_kib / statistics.mean(fetch[copy])
    w_factor = copy_kib / statistics.mean(write[copy])
    f_kib = statistics.mean(fetch[fused])
    w_kib = statistics.mean(write[fused])
    traffic = (f_kib * f_factor + w_kib * w_factor) * 1024
    return {
        "kernel": short_name(fused),
        "workload": "fused gather, TP=8, V=163840, M=256, cap=256, 3 rotating buffer sets",
        "kernel_source_sha256_16": kernel_source_hash(),
        "variant": "fused",
        "copy_kernel_bytes": COPY_BYTES,
        "copy_fetch_kib_per_dispatch": statistics.mean(fetch[copy]),
        "copy_write_kib_per_dispatch": statistics.mean(write[copy]),
        "fetch_scale": f_factor,
        "write_scale": w_factor,
        "fetch_kib_per_dispatch": f_kib,
        "write_kib_per_dispatch": w_kib,
        "dispatches": [len(fetch[fused]), len(write[fused])],
        "traffic_bytes_per_launch": round(traffic),
        "algorithmic_bytes_per_launch": M256_BYTES,
        "traffic_over_algorithmic": traffic / M256_BYTES,
        "commands": [cmd_fetch, cmd_write],
    }


# Derived quantities of the SQ report; the GPU has 8 XCDs of 32 CUs, 4 SIMDs each.
XCDS, SIMDS = 8, 256 * 4


def sq_report(csvs: list[str], kernel: str, commands: list[str]) -> str:
    """Median per-dispatch SQ/TCC/GRBM counters of the kernels whose name
    contains ``kernel``, over several ``--pmc`` runs (one counter set each)."""
    per: dict[str, list[float]] = {}
    durs: list[int] = []
    clocks: list[float] = []  # GHz, GRBM_GUI_ACTIVE / 8 over the same dispatch's duration
    names: set[str] = set()
    for path in csvs:
        seen: set[str] = set()
        for r in csv.DictReader(open(path)):
            if kernel not in r["Kernel_Name"]:
                continue
            names.add(short_name(r["Kernel_Name"]))
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            dt = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                clocks.append(float(r["Counter_Value"]) / XCDS / dt)
            if r["Dispatch_Id"] not in seen:
                seen.add(r["Dispatch_Id"])
                durs.append(dt)
    med = {k: statistics.median(v) for k, v in per.items()}
    dur = statistics.median(durs)
    lines = ["# SQ counters of the M=256 lm_head product (rocprofv3)", "",
             "Kernel " + ", ".join(f"`{n}`" for n in sorted(names)) + ".", "",
             "Commands (TMPDIR=/tmp; paths relative to the repository root):", ""]
    lines += ["    " + c for c in commands]
    lines += ["", f"Median over {len(durs)} profiled dispatches; median duration {dur / 1e3:.1f} us.", "",
              "| counter | median per dispatch |", "|---|---|"]
    lines += [f"| `{k}` | {v:.4g} |" for k, v in sorted(med.items())]
    lines += ["", "Derived (GRBM_GUI_ACTIVE sums its 8 XCD instances):", ""]

    def has(*ks):
        return all(k in med for k in ks)
    if has("GRBM_GUI_ACTIVE"):
        cyc = med["GRBM_GUI_ACTIVE"] / XCDS
        lines.append(f"- shader clock: GRBM_GUI_ACTIVE / 8 / that dispatch's duration = "
                     f"{statistics.median(clocks):.2f} GHz (median)")
        if has("SQ_VALU_MFMA_BUSY_CYCLES"):
            lines.append(f"- MFMA busy per SIMD: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8)"
                         f" = {med['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * cyc) * 100:.1f} %")
    if has("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA"):
        lines.append(f"- busy cycles per MFMA instruction: "
                     f"{med['SQ_VALU_MFMA_BUSY_CYCLES'] / med['SQ_INSTS_MFMA']:.1f}")
    if has("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"):
        lines.append(f"- LDS bank-conflict cycles / LDS active cycles: "
                     f"{med['SQ_LDS_BANK_CONFLICT'] / med['SQ_LDS_IDX_ACTIVE'] * 100:.1f} %")
    if has("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"):
        lines.append(f"- wave time waiting on a counter (any): SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES = "
                     f"{med['SQ_WAIT_INST_ANY'] / med['SQ_WAVE_CYCLES'] * 100:.1f} %")
    if has("SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"):
        lines.append(f"- of which on LDS: SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES = "
                     f"{med['SQ_WAIT_INST_LDS'] / med['SQ_WAVE_CYCLES'] * 100:.1f} %")
    if has("TCC_HIT_sum", "TCC_MISS_sum"):
        lines.append(f"- L2 hit rate: {med['TCC_HIT_sum'] / (med['TCC_HIT_sum'] + med['TCC_MISS_sum']) * 100:.1f} %")
    return "\n".join(lines) + "\n"


def clock_report(csv_path: str, kernel: str, command: str) -> str:
    """Per-dispatch duration, shader clock (GRBM_GUI_ACTIVE / 8 XCDs over the
    dispatch's duration) and MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over
    1024 SIMDs' cycles) of the kernels whose name contains ``kernel``."""
    per: dict[int, dict[str, float]] = {}
    names: set[str] = set()
    for r in csv.DictReader(open(csv_path)):
        if kernel not in r["Kernel_Name"]:
            continue
        names.add(short_name(r["Kernel_Name"]))
        d = per.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    rows = []
    for disp in sorted(per):
        d = per[disp]
        if "GRBM_GUI_ACTIVE" not in d:
            continue
        cyc = d["GRBM_GUI_ACTIVE"] / XCDS
        busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cyc) if "SQ_VALU_MFMA_BUSY_CYCLES" in d else None
        rows.append((disp, d["ns"] / 1e3, cyc / d["ns"], busy))
    lines = ["# Shader clock under back-to-back lm_head products (rocprofv3)", "",
             "Kernel " + ", ".join(f"`{n}`" for n in sorted(names)) + ".", "",
             "Command (TMPDIR=/tmp; paths relative to the repository root):", "", "    " + command, "",
             "| launch | duration us | shader clock GHz | MFMA busy % | duration x clock (k cycles) |",
             "|---|---|---|---|---|"]
    for n, (disp, us, ghz, busy) in enumerate(rows):
        b = f"{busy * 100:.1f}" if busy is not None else "-"
        lines.append(f"| {n + 1} | {us:.1f} | {ghz:.2f} | {b} | {us * ghz:.0f} |")
    if rows:
        us = [r[1] for r in rows]
        ghz = [r[2] for r in rows]
        fast = min(range(len(rows)), key=lambda i: us[i])
        slow = max(range(len(rows)), key=lambda i: us[i])
        lines += ["", f"{len(rows)} dispatches: fastest {us[fast]:.1f} us at {ghz[fast]:.2f} GHz, "
                      f"slowest {us[slow]:.1f} us at {ghz[slow]:.2f} GHz, median "
                      f"{statistics.median(us):.1f} us at {statistics.median(ghz):.2f} GHz."]
    return "\n".join(lines) + "\n"


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("stats_csv")
    k.add_argument("--command", required=True)
    k.add_argument("--out", required=True)
    k.add_argument("--trace", help="the run's *_kernel_trace.csv, for median durations")
    k.add_argument("--json", help="also write the M=1 fused gather's median duration (with the "
                                  "kernel source hash) to this JSON file; needs --trace")
    c = sub.add_parser("counters")
    c.add_argument("fetch_csv")
    c.add_argument("write_csv")
    c.add_argument("--command-fetch", required=True)
    c.add_argument("--command-write", required=True)
    c.add_argument("--out", required=True)
    q = sub.add_parser("sq")
    q.add_argument("csvs", nargs="+", help="*_counter_collection.csv of each --pmc run")
    q.add_argument("--kernel", required=True, help="substring of the kernel name")
    q.add_argument("--command", action="append", required=True)
    q.add_argument("--out", required=True)
    w = sub.add_parser("clock")
    w.add_argument("csv", help="*_counter_collection.csv of the --pmc run")
    w.add_argument("--kernel", required=True, help="substring of the kernel name")
    w.add_argument("--command", required=True)
    w.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.what == "clock":
        text = clock_report(a.csv, a.kernel, a.command)
        open(a.out, "w").write(text)
        print(text)
    elif a.what == "sq":
        text = sq_report(a.csvs, a.kernel, a.command)
        open(a.out, "w").write(text)
        print(text)
    elif a.what == "kernels":
        text = kernels_report(a.stats_csv, a.command, a.trace)
        open(a.out, "w").write(text)
        print(text)
        if a.json:
            m1 = m1_fused_times(a.trace)
            if m1 is None:
                raise SystemExit("no fused gather in the trace")
            split = m1_split_times(a.trace, m1["grid_threads"])
            if split is not None:
                m1["split"] = split
            m1["command"] = a.command
            open(a.json, "w").write(json.dumps(m1, indent=1) + "\n")
            print(json.dumps(m1))
    else:
        rep = counters_report(a.fetch_csv, a.write_csv, a.command_fetch, a.command_write)
        open(a.out, "w").write(json.dumps(rep, indent=1) + "\n")
        md = os.path.splitext(a.out)[0] + ".md"
        open(md, "w").write(
            "# HBM traffic of the M=256 fused gather (rocprofv3 counters)\n\n"
            f"Kernel `{rep['kernel']}`, source hash `{rep['kernel_source_sha256_16']}`.\n\n"
            "Commands (TMPDIR=/tmp; paths relative to the repository root):\n\n"
            + "".join(f"    {cmd}\n" for cmd in rep["commands"]) +
            "\n| | FETCH_SIZE KiB | WRITE_SIZE KiB |\n|---|---|---|\n"
            f"| plain 256 MiB copy (per dispatch) | {rep['copy_fetch_kib_per_dispatch']:.1f} | "
            f"{rep['copy_write_kib_per_dispatch']:.1f} |\n"
            f"| scale to bytes of the copy | x{rep['fetch_scale']:.4f} | x{rep['write_scale']:.4f} |\n"
            f"| fused gather M=256 (per dispatch, {rep['dispatches'][0]} runs) | "
            f"{rep['fetch_kib_per_dispatch']:.1f} | {rep['write_kib_per_dispatch']:.1f} |\n\n"
            f"Traffic per launch: {rep['traffic_bytes_per_launch']:,} B; algorithmic "
            f"{rep['algorithmic_bytes_per_launch']:,} B; ratio {rep['traffic_over_algorithmic']:.3f}.\n")
        print(json.dumps(rep, indent=1))


if __name__ == "__main__":
    main()
