"""Summaries of rocprofv3 runs for the attention kernels (text files under profiles/).

    python -m exact_long_context_cqsa_amd.profiling \
        --name fwd_kernel_causal_n32768_h8_d64_f16 --kernel fwd_ \
        --trace <kernel_trace.csv> --fetch <fetch counter_collection.csv> --write <write counter_collection.csv> \
        --command "<the rocprofv3 command lines that produced the CSVs>"

The kernel trace gives the per-launch duration of the kernel whose name contains --kernel.  With
--copy-trace it summarises the host-to-device streaming of a --memory-copy-trace run instead.  FETCH_SIZE and
WRITE_SIZE (KiB per dispatch) are scaled by what the same counters read for the plain 1 GiB device copy in
the same run (bench.py --copy-calibration), giving HBM bytes per launch.  The summary records the SHA-256 of
the kernel source it measured; bench.py reports the traffic only while the source is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
KERNEL_SOURCE = os.path.join(PKG, "csrc", "cqsa_kernels.hip")
COPY_BYTES = 1 << 30


def kernel_source_sha256() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _grid(r: dict) -> int:
    if r.get("Grid_Size"):
        return int(r["Grid_Size"])
    return int(r.get("Grid_Size_X") or 1) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)


def _pick(rows: list, kernel: str, grid: int | None, select: str | None) -> list:
    """Dispatches of the kernel (name contains `kernel`; grid size `grid` if given), in dispatch order,
    then the python slice `select` ("a:b") of them if given: a way to single out one phase of a run
    whose phases launch the same kernel."""
    got = [r for r in rows if kernel in r.get("Kernel_Name", "") and (grid is None or _grid(r) == grid)]
    got.sort(key=lambda r: int(r.get("Dispatch_Id") or 0))
    if select:
        a, _, b = select.partition(":")
        got = got[int(a) if a else None:int(b) if b else None]
    return got


def trace_stats(path: str, kernel: str, grid: int | None = None, select: str | None = None) -> dict:
    durs = []
    name = None
    for r in _pick(_rows(path), kernel, grid, select):
        durs.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        name = r["Kernel_Name"]
    if not durs:
        raise SystemExit(f"no dispatch of a kernel matching {kernel!r} in {path}")
    return {"kernel_name": name, "calls": len(durs), "avg_ns": statistics.mean(durs), "min_ns": min(durs),
            "max_ns": max(durs), "median_ns": statistics.median(durs)}


def counter_per_dispatch(path: str, counter: str, kernel: str, grid: int | None = None,
                         select: str | None = None) -> tuple[float, float]:
    """(mean value for the measured kernel's dispatches, value for the 1 GiB copy dispatch)."""
    rows = [r for r in _rows(path) if r["Counter_Name"] == counter]
    kvals = [float(r["Counter_Value"]) for r in _pick(rows, kernel, grid, select)]
    # the calibration copy: the runtime's device-to-device copy kernel; a run without one (a copy that
    # torch ran as an elementwise kernel) falls back to the largest elementwise dispatch
    def copies(words):
        return [float(r["Counter_Value"]) for r in rows
                if kernel not in r.get("Kernel_Name", "") and int(r.get("Grid_Size", "0") or 0) > 0
                and any(w in r.get("Kernel_Name", "").lower() for w in words)]
    cvals = copies(("copybuffer",)) or copies(("copy", "elementwise"))
    if not kvals or not cvals:
        raise SystemExit(f"{counter}: kernel or copy dispatch missing in {path}")
    return statistics.mean(kvals), max(cvals)


def summarise(args) -> str:
    grid, select = getattr(args, "grid", None), getattr(args, "select", None)
    csel = getattr(args, "counter_select", None) or select
    ts = trace_stats(args.trace, args.kernel, grid, select)
    fk, fc = counter_per_dispatch(args.fetch, "FETCH_SIZE", args.kernel, grid, csel)
    wk, wc = counter_per_dispatch(args.write, "WRITE_SIZE", args.kernel, grid, csel)
    f_scale = COPY_BYTES / (fc * 1024.0)     # the copy reads 1 GiB
    w_scale = COPY_BYTES / (wc * 1024.0)     # and writes 1 GiB
    fetch_b = fk * 1024.0 * f_scale
    write_b = wk * 1024.0 * w_scale
    sel = []
    if grid or select:
        sel.append(f"dispatches: grid size {grid}" if grid else "dispatches: every grid size")
        if select:
            sel.append(f"selected: [{select}] of the matching dispatches, in dispatch order (kernel trace)")
        if csel != select:
            sel.append(f"selected: [{csel}] of the matching dispatches of the counter runs")
    lines = [
        f"# {args.name}",
        "",
        f"kernel: `{ts['kernel_name']}`",
        *sel,
        f"kernel_source_sha256: {kernel_source_sha256()}",
        "",
        "## Commands",
        "",
        "```",
        args.command.strip(),
        "```",
        "",
        "## Kernel trace (rocprofv3 --kernel-trace --stats)",
        "",
        f"calls: {ts['calls']}",
        f"avg_ns: {ts['avg_ns']:.0f}",
        f"median_ns: {ts['median_ns']:.0f}",
        f"min_ns: {ts['min_ns']}",
        f"max_ns: {ts['max_ns']}",
        "",
        "## HBM traffic (rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE)",
        "",
        f"fetch_kib_per_dispatch: {fk:.1f}  (1 GiB copy reads {fc:.1f} KiB: scale {f_scale:.3f})",
        f"write_kib_per_dispatch: {wk:.1f}  (1 GiB copy writes {wc:.1f} KiB: scale {w_scale:.3f})",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
    ]
    if args.note:
        lines += ["", "## Notes", "", args.note.strip()]
    return "\n".join(lines) + "\n"


def summarise_mfma(args) -> str:
    """Matrix-core counters of one kernel from a run with --kernel-trace and
    --pmc MfmaFlopsF16 MfmaFlopsBF16 MfmaUtil GRBM_GUI_ACTIVE: the FLOPs the MFMA instructions executed
    per launch (against the algorithmic count), the share of SIMD cycles the matrix cores were busy,
    and the clock the launch ran at (GRBM_GUI_ACTIVE summed over the XCDs, per XCD, over the launch's
    duration in the same run)."""
    grid, select = getattr(args, "grid", None), getattr(args, "select", None)
    durs = {int(r["Dispatch_Id"]): int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            for r in _pick(_rows(args.trace), args.kernel, grid, select)}
    per = {}
    for r in _pick(_rows(args.counters), args.kernel, grid, None):
        d = int(r["Dispatch_Id"])
        if d in durs:
            per.setdefault(d, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no counter rows for the selected dispatches of {args.kernel!r}")
    mean = lambda key: statistics.mean(v.get(key, 0.0) for v in per.values())
    flop = mean("MfmaFlopsF16") + mean("MfmaFlopsBF16")
    util = mean("MfmaUtil")
    cyc = mean("GRBM_GUI_ACTIVE") / args.xcds
    avg_ns = statistics.mean(durs[d] for d in per)
    name = next(r["Kernel_Name"] for r in _pick(_rows(args.trace), args.kernel, grid, select))
    lines = [
        f"# {args.name}",
        "",
        f"kernel: `{name}`",
        f"kernel_source_sha256: {kernel_source_sha256()}",
        "",
        "## Commands",
        "",
        "```",
        args.command.strip(),
        "```",
        "",
        "## Matrix-core counters (rocprofv3 --kernel-trace --pmc MfmaFlopsF16 MfmaFlopsBF16 MfmaUtil GRBM_GUI_ACTIVE)",
        "",
        f"calls: {len(per)}",
        f"avg_ns: {avg_ns:.0f}",
        f"mfma_flop_per_launch: {flop:.4e}",
        f"algorithmic_flop_per_launch: {args.algorithmic_flop:.4e}",
        f"executed_over_algorithmic: {flop / args.algorithmic_flop:.4f}",
        f"mfma_util_pct: {util:.1f}",
        f"gui_active_cycles_per_xcd: {cyc:.0f}",
        f"clock_ghz: {cyc / avg_ns:.3f}",
        f"algorithmic_tflops_in_this_run: {args.algorithmic_flop / avg_ns / 1e3:.1f}",
        f"executed_tflops_in_this_run: {flop / avg_ns / 1e3:.1f}",
    ]
    if args.note:
        lines += ["", "## Notes", "", args.note.strip()]
    return "\n".join(lines) + "\n"


WAVE_STATE_PASS1 = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                    "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
WAVE_STATE_PASS2 = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_LDS",
                    "SQ_INSTS_VALU_TRANS_F32", "SQ_ACTIVE_INST_SCA", "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE")


def _pass_means(directory: str, kernel: str, grid, select) -> tuple[dict, list]:
    """Per-dispatch means of every counter of one rocprofv3 --kernel-trace --pmc run (its directory holds
    the run's kernel_trace.csv and counter_collection.csv), over the selected dispatches of the kernel;
    and those dispatches' durations."""
    trace = sorted(glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True))
    ctr = sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True))
    if not trace or not ctr:
        raise SystemExit(f"{directory}: kernel_trace.csv or counter_collection.csv missing")
    durs = {int(r["Dispatch_Id"]): int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            for r in _pick(_rows(trace[0]), kernel, grid, select)}
    per = {}
    for r in _pick(_rows(ctr[0]), kernel, grid, None):
        d = int(r["Dispatch_Id"])
        if d in durs:
            c = per.setdefault(d, {})
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{directory}: no counter rows for the selected dispatches of {kernel!r}")
    names = set().union(*per.values())
    return {n: statistics.mean(v.get(n, 0.0) for v in per.values()) for n in names}, [durs[d] for d in per]


def summarise_wave_state(args) -> str:
    """Where a kernel's waves spend their time, from two rocprofv3 --kernel-trace --pmc runs of the same
    command (WAVE_STATE_PASS1, then WAVE_STATE_PASS2; each counter summed over the chip, per dispatch):
    the shares of the waves' resident cycles spent issuing an instruction (SQ_ACTIVE_INST_ANY), ready but
    waiting for an issue slot (SQ_WAIT_INST_ANY) and waiting on a dependency or barrier (SQ_WAIT_ANY);
    VALUBusy as rocprofv3 defines it for gfx950 (SQ_ACTIVE_INST_VALU per CU over GRBM_GUI_ACTIVE per XCD);
    the matrix cores' busy share of SIMD cycles; and the instructions each wave issued."""
    grid, select = getattr(args, "grid", None), getattr(args, "select", None)
    dirs = [d for d in args.wave_state.split(",") if d]
    if len(dirs) != 2:
        raise SystemExit("--wave-state takes the two run directories, comma-separated")
    a, durs = _pass_means(dirs[0], args.kernel, grid, select)
    b, _ = _pass_means(dirs[1], args.kernel, grid, select)
    cus = args.cus
    cyc = a["GRBM_GUI_ACTIVE"] / args.xcds
    wave = a["SQ_WAVE_CYCLES"]
    waves = b["SQ_WAVES"]
    mfma = b["SQ_INSTS_MFMA"]
    trace = sorted(glob.glob(os.path.join(dirs[0], "**", "*kernel_trace.csv"), recursive=True))[0]
    name = next(r["Kernel_Name"] for r in _pick(_rows(trace), args.kernel, grid, select))
    avg_ns = statistics.mean(durs)
    lines = [
        f"# {args.name}",
        "",
        f"kernel: `{name}`",
        f"kernel_source_sha256: {kernel_source_sha256()}",
        "",
        "## Commands",
        "",
        "```",
        args.command.strip(),
        "```",
        "",
        "## Wave states (rocprofv3 --kernel-trace --pmc, two passes)",
        "",
        f"calls: {len(durs)}",
        f"avg_ns: {avg_ns:.0f}",
        f"gui_active_cycles_per_xcd: {cyc:.0f}",
        f"clock_ghz: {cyc / avg_ns:.3f}",
        f"wave_share_issuing: {a['SQ_ACTIVE_INST_ANY'] / wave:.3f}",
        f"wave_share_waiting_for_issue: {a['SQ_WAIT_INST_ANY'] / wave:.3f}",
        f"wave_share_waiting_on_dependency: {a['SQ_WAIT_ANY'] / wave:.3f}",
        f"wave_share_lds_active: {a['SQ_ACTIVE_INST_LDS'] / wave:.3f}",
        f"valu_busy_pct: {100.0 * a['SQ_ACTIVE_INST_VALU'] / cus / cyc:.1f}",
        f"mfma_busy_pct: {100.0 * a['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * cus) / cyc:.1f}",
        f"waves_per_launch: {waves:.0f}",
        f"valu_insts_per_wave: {b['SQ_INSTS_VALU'] / waves:.1f}  (the MFMA instructions included)",
        f"mfma_insts_per_wave: {mfma / waves:.1f}",
        f"trans_f32_insts_per_wave: {b['SQ_INSTS_VALU_TRANS_F32'] / waves:.1f}",
        f"salu_insts_per_wave: {b['SQ_INSTS_SALU'] / waves:.1f}",
        f"lds_insts_per_wave: {b['SQ_INSTS_LDS'] / waves:.1f}",
        f"per_mfma: valu_other {(b['SQ_INSTS_VALU'] - mfma) / mfma:.2f}, trans {b['SQ_INSTS_VALU_TRANS_F32'] / mfma:.2f}, "
        f"salu {b['SQ_INSTS_SALU'] / mfma:.2f}, lds {b['SQ_INSTS_LDS'] / mfma:.2f}",
    ]
    if args.note:
        lines += ["", "## Notes", "", args.note.strip()]
    return "\n".join(lines) + "\n"


def summarise_copies(args) -> str:
    """Host-to-device streaming from a rocprofv3 --memory-copy-trace run.  The trace gives each copy's
    stream and duration but not its size, so the bytes are the plan's (cqsa_plan_info.h2d_bytes, as the
    run reported them); the achieved rate is those bytes over the summed durations of the copies on the
    library's H2D stream."""
    per = {}
    for r in _rows(args.copy_trace):
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        per.setdefault((r["Direction"], r["Stream_Id"]), []).append(d)
    key = [k for k in per if k[1] == str(args.h2d_stream)]
    if len(key) != 1:
        raise SystemExit(f"expected one direction on stream {args.h2d_stream}: {sorted(per)}")
    durs = per[key[0]]
    total_ns = sum(durs)
    gbs = args.h2d_bytes / total_ns
    lines = [
        f"# {args.name}",
        "",
        "## Commands",
        "",
        "```",
        args.command.strip(),
        "```",
        "",
        "## Copies (rocprofv3 --memory-copy-trace)",
        "",
    ]
    for (direction, stream), v in sorted(per.items()):
        lines.append(f"- stream {stream}, {direction}: {len(v)} copies, {sum(v) / 1e6:.1f} ms in total, "
                     f"longest {max(v) / 1e6:.2f} ms")
    lines += [
        "",
        f"h2d_stream: {args.h2d_stream}",
        f"h2d_copies: {len(durs)}",
        f"h2d_bytes: {args.h2d_bytes}",
        f"h2d_busy_ns: {total_ns}",
        f"h2d_gbs: {gbs:.2f}",
        f"link_peak_gbs: {args.link_gbs:.2f}",
        f"h2d_frac_of_link: {gbs / args.link_gbs:.3f}",
    ]
    if args.note:
        lines += ["", "## Notes", "", args.note.strip()]
    return "\n".join(lines) + "\n"


def read_profile(path: str) -> dict:
    """Key: value pairs of a summary written by this module."""
    out = {}
    if not os.path.exists(path):
        return out
    for ln in open(path):
        m = re.match(r"^([a-z_0-9]+):\s*(\S+)", ln.strip())
        if m:
            out[m.group(1)] = m.group(2)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--name", required=True)
    ap.add_argument("--kernel")
    ap.add_argument("--trace")
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--counters", help="counter_collection.csv with the matrix-core counters: summarise those")
    ap.add_argument("--algorithmic-flop", type=float, default=0.0, help="algorithmic FLOP per launch (--counters)")
    ap.add_argument("--xcds", type=int, default=8, help="XCDs GRBM_GUI_ACTIVE is summed over (--counters)")
    ap.add_argument("--wave-state", default=None,
                    help="the two run directories of the wave-state counter passes, comma-separated: summarise those")
    ap.add_argument("--cus", type=int, default=256, help="compute units of the device (--wave-state)")
    ap.add_argument("--copy-trace", help="memory_copy_trace.csv: summarise the H2D streaming instead")
    ap.add_argument("--h2d-stream", type=int, default=1)
    ap.add_argument("--h2d-bytes", type=int, default=0)
    ap.add_argument("--link-gbs", type=float, default=0.0)
    ap.add_argument("--grid", type=int, default=None, help="only dispatches of this grid size (threads)")
    ap.add_argument("--select", default=None, help="python slice a:b of the matching dispatches")
    ap.add_argument("--counter-select", default=None,
                    help="the slice for the FETCH_SIZE / WRITE_SIZE runs when their command differs (default --select)")
    ap.add_argument("--command", required=True)
    ap.add_argument("--note", default="")
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    if args.wave_state:
        if not args.kernel:
            ap.error("--wave-state needs --kernel")
        text = summarise_wave_state(args)
    elif args.counters:
        if not (args.kernel and args.trace and args.algorithmic_flop > 0):
            ap.error("--counters needs --kernel, --trace and --algorithmic-flop")
        text = summarise_mfma(args)
    elif args.copy_trace:
        if args.h2d_bytes <= 0 or args.link_gbs <= 0:
            ap.error("--copy-trace needs --h2d-bytes and --link-gbs")
        text = summarise_copies(args)
    else:
        if not (args.kernel and args.trace and args.fetch and args.write):
            ap.error("--kernel, --trace, --fetch and --write are required")
        text = summarise(args)
    out = args.out or os.path.join(ROOT, "profiles", args.name + ".md")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
