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


def _medians(trace_csv: str | None) -> dict[str, float]:
    """Median duration (ns) per kernel name from a ``*_kernel_trace.csv``."""
    if not trace_csv:
        return {}
    durs: dict[str, list[int]] = {}
    for r in csv.DictReader(open(trace_csv)):
        durs.setdefault(r["Kernel_Name"], []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return {k: statistics.median(v) for k, v in durs.items()}


def kernels_report(stats_csv: str, command: str, trace_csv: str | None = None) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    med = _medians(trace_csv)
    lines = ["# rocprofv3 kernel summary", "", "Command (TMPDIR=/tmp; paths relative to the repository root):", "",
             "    " + command, "",
             "| kernel | calls | avg us | median us | min us | max us | share |",
             "|---|---|---|---|---|---|---|"]
    for r in rows:
        m = f"{med[r['Name']] / 1e3:.3f}" if r["Name"] in med else "-"
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs'])/1e3:.3f} | "
                     f"{m} | {float(r['MinNs'])/1e3:.3f} | {float(r['MaxNs'])/1e3:.3f} | "
                     f"{float(r['Percentage']):.1f} % |")
    lines += ["", f"Kernel source hash: `{kernel_source_hash()}`", ""]
    # The bench runs the fused gather at M=1 (a few us per call) and at M=256
    # (tens of us); the instantiation (vectors per lane) depends on the size.
    for r in rows:
        n = short_name(r["Name"])
        if not n.startswith("hg::k_fused<"):
            continue
        avg = float(r["AverageNs"]) * 1e-9
        if avg > 20e-6:
            lines.append(f"M=256 fused gather (`{n}`): {float(r['AverageNs'])/1e3:.2f} us average -> "
                         f"{M256_BYTES / avg / 1e9:.1f} GB/s algorithmic "
                         f"({M256_BYTES / avg / 8e12 * 100:.1f} % of 8 TB/s).")
        else:
            m = f", {med[r['Name']] / 1e3:.3f} us median" if r["Name"] in med else ""
            lines.append(f"M=1 fused gather (`{n}`): {float(r['AverageNs'])/1e3:.3f} us average "
                         f"kernel duration{m}, {float(r['MinNs'])/1e3:.3f} us minimum.")
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


def main() -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("stats_csv")
    k.add_argument("--command", required=True)
    k.add_argument("--out", required=True)
    k.add_argument("--trace", help="the run's *_kernel_trace.csv, for median durations")
    c = sub.add_parser("counters")
    c.add_argument("fetch_csv")
    c.add_argument("write_csv")
    c.add_argument("--command-fetch", required=True)
    c.add_argument("--command-write", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.what == "kernels":
        text = kernels_report(a.stats_csv, a.command, a.trace)
        open(a.out, "w").write(text)
        print(text)
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
