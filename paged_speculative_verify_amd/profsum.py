"""Summaries of rocprofv3 output for the kernels of libpta.

Three summaries, all written as short text under ``profiles/``:

* ``trace``: the ``--kernel-trace --stats`` table (calls, mean and total time
  per kernel) of one bench run, as Markdown.
* ``traffic``: HBM bytes per launch of the attention kernel from two ``--pmc``
  runs (``FETCH_SIZE`` and ``WRITE_SIZE``, KiB per dispatch). Each counter is
  scaled by what it reads for a device copy of known size, measured in runs of
  their own (``bench.py --copy-calibration``): on MI355X a 1 GiB copy reads as
  0.5 GiB fetched and 1 GiB written. The JSON twin carries the hash of the
  kernel sources it was taken on, and the bench reports the figure only while
  that hash still matches.
* ``sq``: per-dispatch means of SQ/GRBM counter passes of one kernel and the
  rates derived from them (MFMA busy share of SIMD cycles, MFMA/VALU
  co-execution, bf16 MFMA flop rate, issue and wait shares of wave cycles,
  instructions per MFMA, LDS bank-conflict cycles).

Usage::

    python -m paged_speculative_verify_amd.profsum trace --csv <dir>/run_kernel_stats.csv \
        --title <workload> --command "<rocprofv3 command>" --out profiles/<name>.md
    python -m paged_speculative_verify_amd.profsum traffic --config <workload> \
        --fetch <dir>/run_counter_collection.csv --write <dir>/run_counter_collection.csv \
        --copy-fetch <csv> --copy-write <csv> --command "<commands>" --out-dir profiles
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
KERNEL_SOURCES = ["pta_device.h", "pta_flash.h", "pta_launch.h", "pta_valu.hip", "pta_stream.hip",
                  "pta_tile.hip", "pta_wide.hip", "pta_aux.hip", "pta_api.hip"]
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30                      # bench.py --copy-calibration copies 1 GiB
# every kernel an attention call launches (the balanced entry launches its grid, then
# slice_merge_kernel)
ATTN_KERNELS = ("stream_attn_kernel", "stream_balanced_kernel", "tile_dma_kernel", "tile_balanced_kernel",
                "wide_balanced_kernel", "tile_attn_kernel", "valu_attn_kernel", "slice_merge_kernel")


def kernel_source_hash() -> str:
    """Short hash over every source that goes into the attention kernels."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    """Kernel name without its trailing argument list (rocprofv3 prints demangled names, which
    may hold other parentheses, as in "(anonymous namespace)::k(int)")."""
    name = name.strip('"')
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            if name[i] == ")":
                depth += 1
            elif name[i] == "(":
                depth -= 1
                if depth == 0:
                    return name[:i].rstrip()
    return name


def _is_attention(name: str) -> bool:
    return any(k in name for k in ATTN_KERNELS)


def counter_per_dispatch(path: str, counter: str, want) -> tuple[float, int, str]:
    """Counter value per call: the mean over the dispatches of each kernel whose name
    passes ``want``, summed over those kernels (a call launches each of them once)."""
    vals = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter or not want(row["Kernel_Name"]):
                continue
            vals.setdefault(_short(row["Kernel_Name"]), []).append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for the kernel asked for")
    total = sum(statistics.fmean(v) for v in vals.values())
    return total, min(len(v) for v in vals.values()), " + ".join(sorted(vals))


def cmd_traffic(a) -> int:
    fetch_kib, n_f, kname = counter_per_dispatch(a.fetch, "FETCH_SIZE", _is_attention)
    write_kib, n_w, _ = counter_per_dispatch(a.write, "WRITE_SIZE", _is_attention)
    cf_kib, _, _ = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", lambda n: COPY_KERNEL in n)
    cw_kib, _, _ = counter_per_dispatch(a.copy_write, "WRITE_SIZE", lambda n: COPY_KERNEL in n)
    f_scale = COPY_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_BYTES / (cw_kib * 1024.0)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    rec = {
        "workload": a.config,
        "kernel": kname,
        "dispatches": {"fetch": n_f, "write": n_w},
        "fetch_kib_per_dispatch": round(fetch_kib, 1),
        "write_kib_per_dispatch": round(write_kib, 1),
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": round(cf_kib, 1),
                             "write_kib": round(cw_kib, 1), "fetch_scale": round(f_scale, 4),
                             "write_scale": round(w_scale, 4)},
        "hbm_bytes_per_launch": round(fetch_b + write_b),
        "hbm_fetch_bytes_per_launch": round(fetch_b),
        "hbm_write_bytes_per_launch": round(write_b),
        "kernel_source_hash": kernel_source_hash(),
        "command": a.command,
    }
    os.makedirs(a.out_dir, exist_ok=True)
    with open(os.path.join(a.out_dir, f"traffic_{a.config}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    lines = [
        f"# HBM traffic of {kname} on {a.config}",
        "",
        "Commands:",
        "",
        "```",
        a.command,
        "```",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| calls counted | {n_f} (FETCH_SIZE), {n_w} (WRITE_SIZE) |",
        f"| FETCH_SIZE per call (every kernel of the call) | {fetch_kib:.1f} KiB |",
        f"| WRITE_SIZE per call (every kernel of the call) | {write_kib:.1f} KiB |",
        f"| 1 GiB copy reads as | {cf_kib:.1f} KiB fetched, {cw_kib:.1f} KiB written |",
        f"| scale (fetch, write) | {f_scale:.4f}, {w_scale:.4f} |",
        f"| HBM bytes per launch | {fetch_b + write_b:.4g} ({fetch_b:.4g} read, {write_b:.4g} written) |",
        f"| kernel source hash | {rec['kernel_source_hash']} |",
        "",
    ]
    with open(os.path.join(a.out_dir, f"traffic_{a.config}.md"), "w") as f:
        f.write("\n".join(lines))
    print(json.dumps(rec))
    return 0


def cmd_trace(a) -> int:
    rows = []
    with open(a.csv, newline="") as f:
        for r in csv.DictReader(f):
            rows.append(r)
    lines = [f"# Kernel trace: {a.title}", "", "Command:", "", "```", a.command, "```", ""]
    if a.bench_json and os.path.exists(a.bench_json):
        with open(a.bench_json) as f:
            txt = [ln for ln in f.read().splitlines() if ln.startswith("{")]
        if txt:
            lines += ["Bench line of the same run:", "", "```", txt[-1], "```", ""]
    lines += ["| kernel | calls | mean (us) | min (us) | max (us) | total (ms) | share |",
              "|---|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| {} | {} | {:.2f} | {:.2f} | {:.2f} | {:.3f} | {:.1f}% |".format(
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    lines.append("")
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


# MI355X: 256 compute units in 8 XCDs, 4 SIMDs each; dense bf16 MFMA peak at 2.4 GHz
NUM_CU, NUM_XCD, SIMD_PER_CU = 256, 8, 4
BF16_PEAK_FLOPS = 2.5e15
I8_PEAK_OPS = 5.0e15


def cmd_sq(a) -> int:
    """SQ counter passes of one kernel: per-dispatch means and the derived rates.
    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x CUs x SIMDs per CU)
    (GRBM_GUI_ACTIVE is summed over the XCDs); bf16 MFMA flops = 512 x
    SQ_INSTS_VALU_MFMA_MOPS_BF16."""
    per = {}
    durs = []
    for path in a.csv:
        by_dispatch = {}
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if a.kernel not in r["Kernel_Name"]:
                    continue
                d = by_dispatch.setdefault(r["Dispatch_Id"], {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                d["_dur_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if not by_dispatch:
            raise SystemExit(f"{path}: no dispatch of a kernel matching {a.kernel!r}")
        for d in by_dispatch.values():
            durs.append(d.pop("_dur_ns"))
            for k, v in d.items():
                per.setdefault(k, []).append(v)
    m = {k: statistics.fmean(v) for k, v in per.items()}
    dur_s = statistics.fmean(durs) / 1e9
    derived = []
    if "SQ_VALU_MFMA_BUSY_CYCLES" in m and "GRBM_GUI_ACTIVE" in m:
        gui = m["GRBM_GUI_ACTIVE"] / NUM_XCD
        derived.append(("MFMA busy (of SIMD cycles)", f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * NUM_CU * SIMD_PER_CU):.1f}%"))
        derived.append(("GPU clock while active (GRBM_GUI_ACTIVE per XCD / duration)", f"{gui / dur_s / 1e9:.2f} GHz"))
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in m:
            derived.append(("MFMA and VALU co-executing (of SIMD cycles)",
                            f"{100 * m['SQ_VALU_MFMA_COEXEC_CYCLES'] / (gui * NUM_CU * SIMD_PER_CU):.1f}%"))
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
        fl = 512 * m["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
        derived.append(("bf16 MFMA flops per dispatch (512 x MOPS)", f"{fl:.4g}"))
        derived.append(("bf16 MFMA rate", f"{fl / dur_s / 1e12:.0f} TFLOP/s ({100 * fl / dur_s / BF16_PEAK_FLOPS:.1f}% of 2.5 PFLOP/s)"))
    if "SQ_INSTS_VALU_MFMA_MOPS_I8" in m:
        ops = 512 * m["SQ_INSTS_VALU_MFMA_MOPS_I8"]
        derived.append(("int8 MFMA ops per dispatch (512 x MOPS)", f"{ops:.4g}"))
        derived.append(("int8 MFMA rate", f"{ops / dur_s / 1e12:.0f} TOP/s ({100 * ops / dur_s / I8_PEAK_OPS:.1f}% of 5 POP/s)"))
    if "SQ_WAVE_CYCLES" in m:
        for k, label in (("SQ_ACTIVE_INST_ANY", "wave cycles issuing any instruction"),
                         ("SQ_ACTIVE_INST_VALU", "wave cycles issuing VALU"),
                         ("SQ_WAIT_INST_ANY", "wave cycles waiting for an instruction to issue")):
            if k in m:
                derived.append((label, f"{100 * m[k] / m['SQ_WAVE_CYCLES']:.1f}%"))
    if "SQ_INSTS_MFMA" in m:
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS"):
            if k in m:
                derived.append((f"{k} per MFMA instruction", f"{m[k] / m['SQ_INSTS_MFMA']:.2f}"))
    if "SQ_LDS_BANK_CONFLICT" in m and "GRBM_GUI_ACTIVE" in m:
        gui = m["GRBM_GUI_ACTIVE"] / NUM_XCD
        derived.append(("LDS bank-conflict cycles (of CU cycles)", f"{100 * m['SQ_LDS_BANK_CONFLICT'] / (gui * NUM_CU):.1f}%"))
    lines = [f"# SQ counters: {a.title}", "", "Commands:", "", "```", a.command, "```", "",
             f"Dispatches of the kernel matching `{a.kernel}`: {len(durs)} per pass; mean duration under "
             f"counters {dur_s * 1e6:.1f} us; kernel source hash {kernel_source_hash()}.", "",
             "| counter | mean per dispatch |", "|---|---|"]
    lines += [f"| {k} | {v:.5g} |" for k, v in sorted(m.items())]
    lines += ["", "| derived | value |", "|---|---|"]
    lines += [f"| {k} | {v} |" for k, v in derived]
    lines.append("")
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--config", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"))
    k = sub.add_parser("trace")
    k.add_argument("--csv", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--command", required=True)
    k.add_argument("--bench-json", default=None)
    k.add_argument("--out", required=True)
    q = sub.add_parser("sq", help="SQ counter passes of one kernel -> Markdown summary")
    q.add_argument("--csv", nargs="+", required=True, help="run_counter_collection.csv of each pass")
    q.add_argument("--kernel", required=True, help="substring of the kernel name")
    q.add_argument("--title", required=True)
    q.add_argument("--command", required=True)
    q.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    return {"traffic": cmd_traffic, "trace": cmd_trace, "sq": cmd_sq}[a.cmd](a)


if __name__ == "__main__":
    raise SystemExit(main())
