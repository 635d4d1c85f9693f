"""HBM traffic of a kernel from rocprofv3 counter runs, calibrated by a plain copy.

Two counter runs of the same command (one with ``--pmc FETCH_SIZE``, one with
``--pmc WRITE_SIZE``, both ``--output-format csv``) give KiB per dispatch for
every kernel.  The command also runs a device-to-device copy of a known size
(``bench.py --calib-copy`` copies ``CALIB_BYTES``); the counter value of that
copy kernel divided by its true bytes is the scale factor applied to the
target kernel's reading:

    traffic = FETCH_KiB * 1024 / fetch_scale + WRITE_KiB * 1024 / write_scale

averaged over the target kernel's dispatches.  ``source_digest()`` fingerprints
the kernel sources, so a stored figure can be dropped once they change.

    python -m vlm_shared_prefix_amd.profiling <fetch_dir> <write_dir> <kernel-substring> [out.md [blocks]]

(blocks: only the dispatches of that many workgroups, one launch shape of the kernel)
    python -m vlm_shared_prefix_amd.profiling --stats <kernel_trace_dir> [out.md]
    python -m vlm_shared_prefix_amd.profiling --mfma <MfmaUtil/MfmaFlops counter dir> [out.md]
"""
import csv
import glob
import hashlib
import os
import sys
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
CALIB_BYTES = 512 << 20          # bytes moved by the calibration copy (read once, written once)
COPY_KERNEL = "copyBuffer"       # the runtime's device-to-device copy kernel


def source_digest() -> str:
    """sha256 over the HIP/C++ sources of libjev.so (kernels, ABI, planner)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(os.path.join(HERE, "csrc"))):
        if name.endswith((".hip", ".cpp", ".h")):
            with open(os.path.join(HERE, "csrc", name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _counter_rows(run_dir: str, counter: str, with_blocks: bool = False):
    """[(dispatch id, kernel name, value)] of one counter, in dispatch order (with_blocks: each
    row also carries the dispatch's workgroup count)."""
    paths = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    out = []
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    row = (int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]))
                    if with_blocks:
                        row += (int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])),)
                    out.append(row)
    return sorted(out)


def per_dispatch(run_dir: str, counter: str, substring: str, blocks: Optional[int] = None):
    """Mean counter value over the dispatches of kernels containing `substring` (of `blocks`
    workgroups only, when given: one launch shape) and their count."""
    vals = [r[2] for r in _counter_rows(run_dir, counter, with_blocks=True)
            if substring in r[1] and (blocks is None or r[3] == blocks)]
    if not vals:
        raise ValueError(f"no dispatch of a kernel containing {substring!r} with {counter}"
                         + (f" and {blocks} blocks" if blocks is not None else ""))
    return sum(vals) / len(vals), len(vals)


def calibration_dispatch(run_dir: str, counter: str):
    """Mean counter value of the calibration copies: the copy-kernel dispatches that follow
    the fill of the calibration source (the last elementwise kernel of the run)."""
    rows = _counter_rows(run_dir, counter)
    fills = [d for d, name, _ in rows if "elementwise" in name]
    if not fills:
        raise ValueError("no calibration fill found (run bench.py with --calib-copy)")
    vals = [v for d, name, v in rows if d > fills[-1] and COPY_KERNEL in name]
    if not vals:
        raise ValueError("no calibration copy dispatch after the fill")
    return sum(vals) / len(vals), len(vals)


def summarize(fetch_dir: str, write_dir: str, kernel: str, blocks: Optional[int] = None) -> dict:
    f_copy, _ = calibration_dispatch(fetch_dir, "FETCH_SIZE")
    w_copy, _ = calibration_dispatch(write_dir, "WRITE_SIZE")
    f_k, n_f = per_dispatch(fetch_dir, "FETCH_SIZE", kernel, blocks)
    w_k, n_w = per_dispatch(write_dir, "WRITE_SIZE", kernel, blocks)
    fetch_scale = f_copy * 1024.0 / CALIB_BYTES
    write_scale = w_copy * 1024.0 / CALIB_BYTES
    traffic = f_k * 1024.0 / fetch_scale + w_k * 1024.0 / write_scale
    return {"kernel": kernel, "blocks": blocks, "dispatches": [n_f, n_w], "fetch_kib": f_k, "write_kib": w_k,
            "copy_fetch_kib": f_copy, "copy_write_kib": w_copy, "fetch_scale": fetch_scale,
            "write_scale": write_scale, "traffic_bytes_per_launch": traffic, "source_digest": source_digest()}


def to_markdown(s: dict, command: str = "") -> str:
    lines = [f"# HBM traffic of `{s['kernel']}` (rocprofv3 FETCH_SIZE / WRITE_SIZE)", ""]
    if command:
        lines += ["Commands (one counter per run):", "", "```", command, "```", ""]
    lines += [
        f"- launch shape: {s['blocks']} blocks" if s.get("blocks") else "- launch shape: every dispatch of the kernel",
        f"- dispatches averaged: {s['dispatches'][0]} (FETCH_SIZE run), {s['dispatches'][1]} (WRITE_SIZE run)",
        f"- kernel FETCH_SIZE: {s['fetch_kib']:.1f} KiB/dispatch, WRITE_SIZE: {s['write_kib']:.1f} KiB/dispatch",
        f"- calibration copy of {CALIB_BYTES >> 20} MiB: FETCH_SIZE {s['copy_fetch_kib']:.1f} KiB, "
        f"WRITE_SIZE {s['copy_write_kib']:.1f} KiB -> scale fetch {s['fetch_scale']:.3f}, "
        f"write {s['write_scale']:.3f}",
        f"- traffic_bytes_per_launch: {s['traffic_bytes_per_launch']:.6e}",
        f"- source_digest: {s['source_digest']}",
    ]
    return "\n".join(lines) + "\n"


def stored_traffic(md_path: str):
    """(bytes per launch, digest) from a summary written by to_markdown, or None."""
    if not os.path.exists(md_path):
        return None
    t = d = None
    with open(md_path) as f:
        for line in f:
            if line.startswith("- traffic_bytes_per_launch:"):
                t = float(line.split(":", 1)[1])
            elif line.startswith("- source_digest:"):
                d = line.split(":", 1)[1].strip()
    return None if t is None or d is None else (t, d)


def _short(name: str) -> str:
    n = name.split("(")[0].replace("void ", "").replace("jevk::", "")
    return n[:48]


def kernel_stats_markdown(run_dir: str, title: str, command: str = "", always=("attn_fwd_f16", "attn_merge")) -> str:
    """Per-kernel totals (rocprofv3 --stats) and per-launch-shape medians (kernel trace): the
    top 16 shapes by total time plus every shape of the `always` kernels."""
    stats = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        raise FileNotFoundError(f"no kernel_stats.csv / kernel_trace.csv under {run_dir}")
    lines = [f"# {title}", ""]
    if command:
        lines += ["Command (from the repository root):", "", "```", command, "```", ""]
    lines += ["Per kernel (durations in microseconds):", "",
              "| kernel | calls | total ms | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    with open(stats[0]) as f:
        for r in csv.DictReader(f):
            lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    groups = {}
    with open(trace[0]) as f:
        for r in csv.DictReader(f):
            key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])),
                   int(r["Grid_Size_Y"]), int(r["Grid_Size_Z"]))
            groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    tot = sum(sum(v) for v in groups.values())
    lines += ["", "Per launch shape (blocks x, y, z), top 16 by total time, then every shape of "
              + " / ".join(f"`{a}`" for a in always) + ":", "",
              "| kernel | blocks | launches | median us | total ms | % |", "|---|---|---|---|---|---|"]
    ranked = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    shown = ranked[:16] + [kv for kv in ranked[16:] if any(a in kv[0][0] for a in always)]
    for (n, gx, gy, gz), v in shown:
        v.sort()
        lines.append(f"| {n} | {gx}x{gy}x{gz} | {len(v)} | {v[len(v) // 2]:.1f} | {sum(v) / 1e3:.2f} | "
                     f"{100 * sum(v) / tot:.1f} |")
    return "\n".join(lines) + "\n"


MFMA_COUNTERS = ("MfmaUtil", "MfmaFlopsF16", "MfmaFlopsBF16")


def mfma_markdown(run_dir: str, title: str, command: str = "",
                  kernels=("attn_fwd_f16", "gemm_bf16w", "gemm_bf16s", "gemm_skinny")) -> str:
    """Per kernel and launch shape: mean MfmaUtil (percent of SIMD cycles with the MFMA unit
    busy) and executed MFMA flops per dispatch (f16 + bf16) from one counter run."""
    paths = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = {}
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] not in MFMA_COUNTERS or not any(k in r["Kernel_Name"] for k in kernels):
                    continue
                blocks = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
                key = (_short(r["Kernel_Name"]), blocks)
                d = per.setdefault(key, {})
                d.setdefault(r["Counter_Name"], {})[int(r["Dispatch_Id"])] = float(r["Counter_Value"])
    lines = [f"# {title}", ""]
    if command:
        lines += ["Command (from the repository root):", "", "```", command, "```", ""]
    lines += ["| kernel | blocks | dispatches | MfmaUtil % | executed MFMA GFLOP / dispatch (f16 + bf16) |",
              "|---|---|---|---|---|"]
    for (name, blocks), d in sorted(per.items(), key=lambda kv: (kv[0][0], -kv[0][1])):
        util = d.get("MfmaUtil", {})
        n = len(util)
        f16 = d.get("MfmaFlopsF16", {})
        b16 = d.get("MfmaFlopsBF16", {})
        fl = [(f16.get(i, 0.0) + b16.get(i, 0.0)) for i in util]
        lines.append(f"| {name} | {blocks} | {n} | {sum(util.values()) / max(1, n):.1f} | "
                     f"{sum(fl) / max(1, n) / 1e9:.2f} |")
    return "\n".join(lines) + "\n"


LDS_TA_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES",
                   "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE", "TA_TA_BUSY_sum", "TA_FLAT_READ_WAVEFRONTS_sum")


def lds_ta_markdown(run_dir: str, title: str, command: str = "", kernels=("attn_fwd_f16", "gemm_bf16w"),
                    xcds: int = 8, cus: int = 256) -> str:
    """Per kernel and launch shape, from one counter run: LDS bank conflicts per LDS-active
    cycle, the fraction of wave cycles spent waiting on LDS instructions, and the texture
    address (TA) units' busy fraction.  GRBM_GUI_ACTIVE reads as the sum over the XCDs and
    TA_TA_BUSY_sum as the sum over the CUs' TA units, so TA busy = TA_TA_BUSY_sum /
    (GRBM_GUI_ACTIVE / xcds * cus)."""
    paths = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = {}
    for p in paths:
        with open(p) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] not in LDS_TA_COUNTERS or not any(k in r["Kernel_Name"] for k in kernels):
                    continue
                blocks = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
                d = per.setdefault((_short(r["Kernel_Name"]), blocks), {})
                c = d.setdefault(r["Counter_Name"], {})
                c[int(r["Dispatch_Id"])] = c.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    lines = [f"# {title}", ""]
    if command:
        lines += ["Command (from the repository root):", "", "```", command, "```", ""]
    lines += ["| kernel | blocks | dispatches | LDS bank conflicts / LDS-active cycle | LDS wait / wave cycle | "
              "TA busy | TA read wavefronts / dispatch |", "|---|---|---|---|---|---|---|"]

    def mean(d, k):
        v = d.get(k, {})
        return sum(v.values()) / max(1, len(v))

    for (name, blocks), d in sorted(per.items(), key=lambda kv: (kv[0][0], -kv[0][1])):
        n = len(d.get("GRBM_GUI_ACTIVE", {}))
        gui = mean(d, "GRBM_GUI_ACTIVE")
        conf = mean(d, "SQ_LDS_BANK_CONFLICT") / max(1.0, mean(d, "SQ_LDS_IDX_ACTIVE"))
        wait = mean(d, "SQ_WAIT_INST_LDS") / max(1.0, mean(d, "SQ_WAVE_CYCLES"))
        ta = mean(d, "TA_TA_BUSY_sum") / max(1.0, gui / xcds * cus)
        lines.append(f"| {name} | {blocks} | {n} | {conf:.3f} | {wait:.3f} | {ta:.2f} | "
                     f"{mean(d, 'TA_FLAT_READ_WAVEFRONTS_sum'):.0f} |")
    return "\n".join(lines) + "\n"


def _with_notes(md: str) -> str:
    """The summary followed by the notes in JEV_STATS_NOTES (which launch shape is which call)."""
    notes = os.environ.get("JEV_STATS_NOTES", "").strip()
    return md + ("\n" + notes + "\n" if notes else "")


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "--lds-ta":
        md = _with_notes(lds_ta_markdown(sys.argv[2], os.environ.get("JEV_STATS_TITLE", "rocprofv3 LDS and TA counters"),
                                         os.environ.get("JEV_STATS_COMMAND", "")))
        if len(sys.argv) > 3:
            with open(sys.argv[3], "w") as f:
                f.write(md)
        print(md)
        sys.exit(0)
    if len(sys.argv) >= 3 and sys.argv[1] == "--mfma":
        md = _with_notes(mfma_markdown(sys.argv[2], os.environ.get("JEV_STATS_TITLE", "rocprofv3 MFMA counters"),
                                       os.environ.get("JEV_STATS_COMMAND", "")))
        if len(sys.argv) > 3:
            with open(sys.argv[3], "w") as f:
                f.write(md)
        print(md)
        sys.exit(0)
    if len(sys.argv) >= 3 and sys.argv[1] == "--stats":
        # JEV_STATS_ALWAYS: comma-separated kernel names whose every launch shape is listed
        always = tuple(a for a in os.environ.get("JEV_STATS_ALWAYS", "attn_fwd_f16,attn_merge").split(",") if a)
        md = _with_notes(kernel_stats_markdown(sys.argv[2],
                                               os.environ.get("JEV_STATS_TITLE", "rocprofv3 kernel statistics"),
                                               os.environ.get("JEV_STATS_COMMAND", ""), always))
        if len(sys.argv) > 3:
            with open(sys.argv[3], "w") as f:
                f.write(md)
        print(md)
        sys.exit(0)
    if len(sys.argv) < 4:
        print(__doc__)
        sys.exit(2)
    # FETCH_DIR WRITE_DIR KERNEL [OUT.md [BLOCKS]]
    s = summarize(sys.argv[1], sys.argv[2], sys.argv[3], int(sys.argv[5]) if len(sys.argv) > 5 else None)
    md = to_markdown(s, os.environ.get("JEV_PMC_COMMAND", ""))
    if len(sys.argv) > 4:
        with open(sys.argv[4], "w") as f:
            f.write(md)
    print(md)
