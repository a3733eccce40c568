"""Summaries of rocprofv3 output for the ``profiles/`` folder.

Two reports, each written as a short Markdown file (and, for the HBM
traffic, a JSON record that ``bench.py`` reads):

* ``trace``: per-kernel launch counts and durations from
  ``rocprofv3 --kernel-trace --stats --output-format csv`` (the
  ``*_kernel_stats.csv`` file), next to the live figures of the bench JSON
  line printed by the same command.
* ``traffic``: HBM bytes per launch from two ``rocprofv3 --pmc`` runs of
  ``bench.py --probe`` (``FETCH_SIZE``, then ``WRITE_SIZE``, KiB per
  dispatch).  Each counter is scaled by the factor that maps its reading for
  the probe's plain device copy of known size to the true byte count.
* ``counters``: per kernel (its last, warmed-up dispatch), the matrix-core
  busy share, the clock, vector instructions per matrix product, LDS bank
  conflicts and HBM GB/s, from two ``rocprofv3 --kernel-trace --stats --pmc``
  runs of a short bench (``SQ_*`` counters; durations from the same runs'
  kernel traces) and the traffic runs.

Usage::

    python -m exact_io_aware_26_amd.profiling trace --stats DIR --bench-json FILE --command CMD --out FILE.md
    python -m exact_io_aware_26_amd.profiling traffic --fetch DIR --write DIR --kernel NAME \\
        --copy-bytes N --commands CMD1 CMD2 --out-json FILE.json --out-md FILE.md
    python -m exact_io_aware_26_amd.profiling counters --pmc DIR_A DIR_B --fetch DIR --write DIR \\
        --copy-bytes N --commands CMD_A CMD_B --out FILE.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = [os.path.join(ROOT, "exact_io_aware_26_amd", "csrc", f)
                  for f in ("fa2_bwd.hip", "fa2_device.h", "fa2_kernels.h")]
COPY_KERNEL = "copyBuffer"     # the runtime's device-to-device copy (torch's copy_ of a uint8 tensor)


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace runs collapsed."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_digest() -> str:
    """sha256 of the code (comments and layout ignored) of the backward kernels'
    sources: what the traffic record was taken on."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def short_name(name: str) -> str:
    m = re.search(r"::(\w+<[^>]*>)", name)
    if m:
        return m.group(1)
    m = re.search(r"(\w*copyBuffer\w*)", name)
    return m.group(1) if m else name[:60]


def _one_csv(directory: str, pattern: str) -> str:
    files = glob.glob(os.path.join(directory, "**", pattern), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one {pattern} under {directory}, found {files}")
    return files[0]


def read_counter(directory: str, counter: str) -> dict[str, list[float]]:
    """Counter values (KiB) per kernel short name, one entry per dispatch."""
    out: dict[str, list[float]] = {}
    with open(_one_csv(directory, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                out.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def traffic(fetch_dir: str, write_dir: str, kernel: str, copy_bytes: int, commands: list[str]):
    fetch = read_counter(fetch_dir, "FETCH_SIZE")
    write = read_counter(write_dir, "WRITE_SIZE")
    copy_names = [k for k in fetch if COPY_KERNEL in k]
    if not copy_names:
        raise SystemExit("the copy probe kernel is missing from the counter runs")
    ck = copy_names[0]
    fetch_scale = copy_bytes / (fetch[ck][0] * 1024.0)
    write_scale = copy_bytes / (write[ck][0] * 1024.0)
    rows = []
    for name in fetch:
        if name not in write:
            continue
        f_kib, w_kib = fetch[name][0], write[name][0]
        rows.append((name, f_kib, w_kib, f_kib * 1024 * fetch_scale, w_kib * 1024 * write_scale))
    target = [r for r in rows if r[0] == kernel]
    if not target:
        raise SystemExit(f"kernel {kernel} not found; have {[r[0] for r in rows]}")
    _, f_kib, w_kib, fb, wb = target[0]
    record = {
        "kernel": kernel,
        "bytes_per_launch": fb + wb,
        "read_bytes": fb,
        "write_bytes": wb,
        "fetch_kib": f_kib,
        "write_kib": w_kib,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "copy_probe_bytes": copy_bytes,
        "source_sha256": kernel_source_digest(),
        "commands": commands,
    }
    md = [f"# HBM traffic per launch, {kernel} and the other kernels of one step", "",
          "Two `rocprofv3 --pmc` runs of `bench.py --probe` (one plain device copy of",
          f"{copy_bytes} bytes, then one forward and each backward stage once), made by:", ""]
    md += [f"    {c}" for c in commands]
    md += ["", f"Calibration on the copy: FETCH_SIZE read {fetch[ck][0]:.1f} KiB and WRITE_SIZE "
           f"{write[ck][0]:.1f} KiB for {copy_bytes / 1024:.0f} KiB moved each way, so reads are scaled by "
           f"{fetch_scale:.4f} and writes by {write_scale:.4f}.", "",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes (scaled) | write bytes (scaled) |",
           "|---|---:|---:|---:|---:|"]
    for name, fk, wk, rb, wbb in rows:
        md.append(f"| {name} | {fk:.1f} | {wk:.1f} | {rb:.4g} | {wbb:.4g} |")
    md += ["", f"Kernel sources sha256: `{record['source_sha256']}`."]
    return record, "\n".join(md) + "\n"


def trace(stats_dir: str, bench_json: str, command: str) -> str:
    with open(_one_csv(stats_dir, "*kernel_stats.csv")) as f:
        stats = list(csv.DictReader(f))
    with open(bench_json) as f:
        line = json.loads([l for l in f.read().splitlines() if l.startswith("{")][-1])
    # Per-dispatch durations, to average the launches of the timed steps only.
    steps = int(line.get("steps", 0))
    per_kernel: dict[str, list[float]] = {}
    with open(_one_csv(stats_dir, "*kernel_trace.csv")) as f:
        for r in sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"])):
            per_kernel.setdefault(short_name(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    md = ["# Kernel trace, one bench run", "", "Made by:", "", f"    {command}", "",
          f"| kernel | launches | average us | min us | max us | share of GPU time | average us, last {steps} |",
          "|---|---:|---:|---:|---:|---:|---:|"]
    for r in stats:
        name = short_name(r["Name"])
        d = per_kernel.get(name, [])[-steps:] if steps else []
        tail = f"{sum(d) / len(d):.1f}" if d else "-"
        md.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                  f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% | {tail} |")
    rf = line.get("roofline", {})
    md += ["", "Live figures printed by the same process (HIP events around each launch on its stream,",
           "averaged over the timed steps; compare with the last column):", "",
           f"- {rf.get('kernel', '?')}: {rf.get('avg_launch_ms', float('nan')) * 1e3:.1f} us per launch, "
           f"{rf.get('achieved', float('nan')):.1f} {rf.get('unit', '')} ({100 * rf.get('frac', float('nan')):.1f}% of peak)",
           f"- forward {line.get('fwd_ms', float('nan')) * 1e3:.1f} us, backward stages "
           + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in line.get("bwd_stage_ms", {}).items()),
           f"- step {line.get('ms_per_step', float('nan')):.3f} ms, {line.get('value', float('nan')):.1f} "
           f"{line.get('unit', '')}"]
    return "\n".join(md) + "\n"


# MI355X: 8 XCDs x 4 shader engines; 256 CUs x 4 SIMDs; a v_mfma_f32_32x32x16_bf16
# keeps a SIMD's matrix core busy for 32 clocks (32768 FLOP).
N_SE, N_SIMD, MFMA_CLOCKS, FLOP_PER_SIMD_CLOCK = 32, 1024, 32, 1024


def _durations_us(directory: str) -> dict[str, float]:
    """Duration of each kernel's last dispatch (the warmed-up one), from the kernel trace."""
    out: dict[str, float] = {}
    with open(_one_csv(directory, "*kernel_trace.csv")) as f:
        for r in sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"])):
            out[short_name(r["Kernel_Name"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    return out


def counters(pmc_dirs: list[str], fetch_dir: str, write_dir: str, copy_bytes: int, commands: list[str]) -> str:
    vals: dict[str, dict[str, float]] = {}
    dur: dict[str, float] = {}
    for d in pmc_dirs:
        with open(_one_csv(d, "*counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                vals.setdefault(short_name(r["Kernel_Name"]), {})[r["Counter_Name"]] = float(r["Counter_Value"])
        for k, v in _durations_us(d).items():
            dur.setdefault(k, v)
    fetch = read_counter(fetch_dir, "FETCH_SIZE")
    write = read_counter(write_dir, "WRITE_SIZE")
    ck = [k for k in fetch if COPY_KERNEL in k][0]
    fs, ws = copy_bytes / (fetch[ck][0] * 1024.0), copy_bytes / (write[ck][0] * 1024.0)
    md = ["# Matrix-core, vector, LDS and HBM counters per kernel (B4 H16 N8192 d128 causal)", "",
          "Counter runs; each kernel's last dispatch (counters and duration from the same run):", ""]
    md += [f"    {c}" for c in commands]
    md += ["", "Derived per kernel: clock = SQ_BUSY_CYCLES / (32 shader engines x duration); MFMA busy = "
           "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x clock x duration); the matrix-core peak at that clock is "
           "1024 SIMDs x clock x 1024 FLOP; VALU/MFMA = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA; "
           "LDS conflicts = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; LDS wait = SQ_WAIT_INST_LDS / "
           "SQ_WAVE_CYCLES; HBM GB/s = (FETCH_SIZE x %.4f + WRITE_SIZE x %.4f) KiB / duration "
           "(scales from a plain copy, as in the traffic record)." % (fs, ws), "",
           "| kernel | us | clock GHz | MFMA busy | VALU per MFMA | LDS bank conflicts | LDS wait | HBM GB/s |",
           "|---|---:|---:|---:|---:|---:|---:|---:|"]
    raw = ["", "Raw counters:", "", "| kernel | counter | value |", "|---|---|---:|"]
    for name, c in vals.items():
        if COPY_KERNEL in name or "FillFunctor" in name or name not in dur:
            continue
        t = dur[name] * 1e-6
        clock = c.get("SQ_BUSY_CYCLES", 0.0) / N_SE / t if t else 0.0
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (N_SIMD * clock * t) if clock else 0.0
        mf = c.get("SQ_INSTS_MFMA", 0.0)
        vpm = (c.get("SQ_INSTS_VALU", 0.0) - mf) / mf if mf else float("nan")
        lds = c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_LDS_IDX_ACTIVE"] if c.get("SQ_LDS_IDX_ACTIVE") else 0.0
        lw = c.get("SQ_WAIT_INST_LDS", 0.0) / c["SQ_WAVE_CYCLES"] if c.get("SQ_WAVE_CYCLES") else 0.0
        hbm = ((fetch.get(name, [0.0])[0] * fs + write.get(name, [0.0])[0] * ws) * 1024.0) / t / 1e9
        md.append(f"| {name} | {dur[name]:.1f} | {clock / 1e9:.2f} | {100 * busy:.1f} % | {vpm:.2f} | "
                  f"{100 * lds:.2f} % | {100 * lw:.1f} % | {hbm:.0f} |")
        for cn in sorted(c):
            raw.append(f"| {name} | {cn} | {c[cn]:.6g} |")
    return "\n".join(md + raw) + "\n"


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--stats", required=True)
    t.add_argument("--bench-json", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    x = sub.add_parser("traffic")
    x.add_argument("--fetch", required=True)
    x.add_argument("--write", required=True)
    x.add_argument("--kernel", required=True)
    x.add_argument("--copy-bytes", type=int, required=True)
    x.add_argument("--commands", nargs="+", required=True)
    x.add_argument("--out-json", required=True)
    x.add_argument("--out-md", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--pmc", nargs="+", required=True)
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--commands", nargs="+", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args()
    if a.what == "counters":
        with open(a.out, "w") as f:
            f.write(counters(a.pmc, a.fetch, a.write, a.copy_bytes, a.commands))
        return
    if a.what == "trace":
        with open(a.out, "w") as f:
            f.write(trace(a.stats, a.bench_json, a.command))
    else:
        rec, md = traffic(a.fetch, a.write, a.kernel, a.copy_bytes, a.commands)
        with open(a.out_json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        with open(a.out_md, "w") as f:
            f.write(md)


if __name__ == "__main__":
    main()
