"""Summaries of rocprofv3 output for the committed profile records.

    python -m entropic_ot_attention_amd.profiling stats <kernel_stats.csv> <out.md> "<command>"
    python -m entropic_ot_attention_amd.profiling traffic <fetch.csv> <write.csv> <out.json> \
        <kernel substring> <calibration kernel substring> <calibration bytes> "<command>" <workload>
    python -m entropic_ot_attention_amd.profiling counters <out.md> "<commands>" <counters.csv> ...
    python -m entropic_ot_attention_amd.profiling mem-counters <out.md> "<commands>" <counters.csv> ...
    python -m entropic_ot_attention_amd.profiling step-counters <out.json> <kernel substring> \
        <workload> <record .md> <counters.csv> ...

`stats` writes a short markdown table (calls, average and total duration per kernel) from a
`--kernel-trace --stats --output-format csv` run.  `traffic` turns two `--pmc FETCH_SIZE` and
`--pmc WRITE_SIZE` runs into HBM bytes per launch of one kernel, each counter scaled by what it
reads for the calibration kernel in the same run (an elementwise kernel that reads and writes a
known number of bytes, bench.py --calibration-copy-mib), and records the workload and a SHA-256
over everything the kernel's machine code is built from (its source, the device and internal
headers it includes, the compiler flags), so a reader can tell when the record no longer
describes the code.
"""

from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
STEP_KERNEL_SOURCES = [os.path.join(PKG, "csrc", f)
                       for f in ("ska_fused.hip", "ska_device.h", "ska_internal.h",
                                 "ska_geometry.cpp")]


def source_sha(paths=None) -> str:
    """SHA-256 over the step kernel's source files and the library's compiler flags."""
    from .build_lib import HIPCC_FLAGS
    h = hashlib.sha256()
    for path in paths or STEP_KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(HIPCC_FLAGS).encode())
    return h.hexdigest()


def stats_markdown(csv_path: str, out_md: str, command: str, top: int = 14) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [
        "# rocprofv3 kernel statistics",
        "",
        "Command:",
        "",
        "```",
        command,
        "```",
        "",
        "| kernel | calls | avg us | total ms | % |",
        "|---|---:|---:|---:|---:|",
    ]
    for r in rows[:top]:
        lines.append(f"| `{r['Name'][:96]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.1f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


# MI355X: 8 XCDs, 256 CUs, 4 SIMDs per CU (GRBM_GUI_ACTIVE is summed over the XCDs; the SQ
# counters over every SIMD).
N_XCD, N_SIMD = 8, 256 * 4


def _per_kernel(csv_paths):
    """kernel name -> counter -> [value per dispatch], over one or more `--pmc` runs."""
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in csv_paths:
        disp = collections.defaultdict(lambda: collections.defaultdict(float))
        names = {}
        for r in csv.DictReader(open(path)):
            disp[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
        for d, cs in disp.items():
            for c, v in cs.items():
                per[names[d]][c].append(v)
    return per


def counters_markdown(csv_paths, out_md: str, command: str, regex_note: str = "") -> None:
    """Per-kernel averages of SQ counters over the dispatches of one or more `--pmc` runs, with
    the unit utilisations derived from them:
      kernel cycles = GRBM_GUI_ACTIVE / 8 XCDs;
      VALU busy = 4 SQ_ACTIVE_INST_VALU / (1024 SIMDs x cycles)   (quad-cycle units);
      LDS busy  = 4 SQ_ACTIVE_INST_LDS / (1024 SIMDs x cycles);
      MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles)."""
    per = _per_kernel(csv_paths)
    lines = ["# rocprofv3 SQ counters", "", "Commands (one counter pass each):", "", "```",
             command, "```", ""]
    if regex_note:
        lines += [regex_note, ""]
    for name in sorted(per, key=lambda k: -sum(per[k].get("GRBM_GUI_ACTIVE", [0]))):
        m = {c: sum(v) / len(v) for c, v in per[name].items()}
        cyc = m.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        w = m.get("SQ_WAVES", 0.0)
        lines += [f"## `{name[:96]}`", "",
                  f"dispatches averaged: {len(per[name].get('GRBM_GUI_ACTIVE', []))}; "
                  f"kernel cycles {cyc:.0f} ({cyc / 2.4e3:.1f} us at 2.4 GHz)", "",
                  "| quantity | value |", "|---|---:|"]
        if w:
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
                      "SQ_INSTS_SALU"):
                if c in m:
                    lines.append(f"| {c} per wave | {m[c] / w:.0f} |")
            lines.append(f"| waves | {w:.0f} |")
        if cyc:
            for label, c, k in (("VALU busy", "SQ_ACTIVE_INST_VALU", 4.0),
                                ("LDS busy", "SQ_ACTIVE_INST_LDS", 4.0),
                                ("MFMA busy", "SQ_VALU_MFMA_BUSY_CYCLES", 1.0)):
                if c in m:
                    lines.append(f"| {label} | {k * m[c] / (N_SIMD * cyc):.3f} |")
        for c in ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"):
            if c in m and cyc:
                lines.append(f"| {c} / (256 CUs x cycles) | {m[c] / (256 * cyc):.3f} |")
        lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


# MI355X L2: 16 channels per XCD, each taking one 128-byte request per cycle.
N_L2_CHANNELS, L2_LINE = 16 * N_XCD, 128


def memory_counters_markdown(csv_paths, out_md: str, command: str) -> None:
    """Per-kernel averages of the cache counters over the dispatches of `--pmc` runs:
      kernel cycles    = GRBM_GUI_ACTIVE / 8 XCDs;
      L2 requests      = TCC_REQ_sum per launch, and per kernel cycle against the 128 channels;
      L2 hit rate      = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum);
      L1 hit rate      = 1 - TCP_TCC_READ_REQ_sum / TCP_TOTAL_CACHE_ACCESSES_sum;
      address unit     = TA_BUSY_avr and TA_BUSY_max over the CUs, per kernel cycle;
      L1 pending stall = TCP_PENDING_STALL_CYCLES_sum / (256 CUs x cycles).
    TCC_BUSY counts a channel busy while it waits on the fabric too, so it is no measure of the
    L2's own load; it is listed as read."""
    per = _per_kernel(csv_paths)
    lines = ["# rocprofv3 cache counters", "", "Commands (one counter pass each):", "", "```",
             command, "```", "",
             "L2 requests are 128-byte lines; the L2 has 16 channels per XCD, 128 in all, each "
             "taking one request per cycle.", ""]
    for name in sorted(per, key=lambda k: -sum(per[k].get("GRBM_GUI_ACTIVE", [0]))):
        m = {c: sum(v) / len(v) for c, v in per[name].items()}
        cyc = m.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        n = min(len(v) for v in per[name].values())
        lines += [f"## `{name[:96]}`", "",
                  f"dispatches averaged per pass: {n}; kernel cycles {cyc:.0f}", "",
                  "| quantity | value |", "|---|---:|"]
        req = m.get("TCC_REQ_sum")
        if req is not None:
            lines.append(f"| L2 requests per launch | {req:.4g} ({req * L2_LINE / 1e9:.3f} GB) |")
            if cyc:
                lines.append(f"| L2 requests per cycle | {req / cyc:.1f} "
                             f"({req / cyc / N_L2_CHANNELS:.3f} of the channels' rate) |")
        if "TCC_HIT_sum" in m and "TCC_MISS_sum" in m:
            tot = m["TCC_HIT_sum"] + m["TCC_MISS_sum"]
            if tot:
                lines.append(f"| L2 hit rate | {m['TCC_HIT_sum'] / tot:.3f} |")
        if "TCP_TOTAL_CACHE_ACCESSES_sum" in m and "TCP_TCC_READ_REQ_sum" in m:
            acc = m["TCP_TOTAL_CACHE_ACCESSES_sum"]
            lines.append(f"| L1 accesses per launch | {acc:.4g} |")
            if acc:
                lines.append(f"| L1 hit rate (reads sent on to L2) | "
                             f"{1 - m['TCP_TCC_READ_REQ_sum'] / acc:.3f} |")
        if cyc:
            for label, c, k in (("address unit busy (mean CU)", "TA_BUSY_avr", 1.0),
                                ("address unit busy (busiest CU)", "TA_BUSY_max", 1.0),
                                ("L1 pending-request stall per CU", "TCP_PENDING_STALL_CYCLES_sum",
                                 1.0 / 256)):
                if c in m:
                    lines.append(f"| {label} | {k * m[c] / cyc:.3f} |")
        if m.get("TCC_CYCLE_sum") and "TCC_BUSY_sum" in m:
            lines.append(f"| TCC_BUSY / TCC_CYCLE | {m['TCC_BUSY_sum'] / m['TCC_CYCLE_sum']:.3f} |")
        lines.append("")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def kernel_busy(csv_paths, kernel: str) -> dict:
    """Busy fractions (as in counters_markdown) averaged over every dispatch of the kernels whose
    name contains `kernel`, across the counter passes."""
    sums = collections.defaultdict(float)
    counts = collections.defaultdict(int)
    for path in csv_paths:
        disp = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"]:
                disp[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        for cs in disp.values():
            for c, v in cs.items():
                sums[c] += v
                counts[c] += 1
    m = {c: sums[c] / counts[c] for c in sums}
    cyc = m.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
    if not cyc:
        raise RuntimeError(f"no GRBM_GUI_ACTIVE for '{kernel}'")
    out = {"cycles": cyc}
    for label, c, k in (("valu_busy", "SQ_ACTIVE_INST_VALU", 4.0),
                        ("lds_busy", "SQ_ACTIVE_INST_LDS", 4.0),
                        ("mfma_busy", "SQ_VALU_MFMA_BUSY_CYCLES", 1.0)):
        out[label] = round(k * m[c] / (N_SIMD * cyc), 4) if c in m else None
    w = m.get("SQ_WAVES", 0.0)
    out["waves"] = round(w) if w else None
    out["valu_insts_per_wave"] = round(m["SQ_INSTS_VALU"] / w) if w and "SQ_INSTS_VALU" in m else None
    out["trans_insts_per_wave"] = (round(m["SQ_INSTS_VALU_TRANS_F32"] / w)
                                   if w and "SQ_INSTS_VALU_TRANS_F32" in m else None)
    return out


def _per_dispatch(csv_path: str, counter: str):
    """{dispatch id: (kernel name, summed counter value)} for one counter."""
    out = collections.defaultdict(lambda: ["", 0.0])
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        d = out[r["Dispatch_Id"]]
        d[0] = r["Kernel_Name"]
        d[1] += float(r["Counter_Value"])
    return out


def traffic_record(fetch_csv: str, write_csv: str, kernel: str, calib_kernel: str, calib_bytes: int,
                   command: str, workload: str):
    rec = {"kernel": kernel, "workload": workload, "source_sha256": source_sha(), "command": command,
           "calibration_kernel": calib_kernel, "calibration_bytes": calib_bytes}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        disp = _per_dispatch(path, counter)
        copies = [v for k, (n, v) in disp.items() if calib_kernel in n]
        kvals = [v for k, (n, v) in disp.items() if kernel in n]
        if not copies or not kvals:
            raise RuntimeError(f"{counter}: calibration copy or kernel '{kernel}' not found")
        copy_kib = max(copies)
        scale = calib_bytes / (copy_kib * 1024.0)        # true bytes per counted byte
        rec[f"{name}_kib_per_launch_raw"] = sum(kvals) / len(kvals)
        rec[f"{name}_calibration_kib"] = copy_kib
        rec[f"{name}_scale"] = scale
        rec[f"{name}_bytes_per_launch"] = sum(kvals) / len(kvals) * 1024.0 * scale
        rec[f"{name}_launches"] = len(kvals)
    rec["bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    return rec


def main(argv):
    if argv[1] == "stats":
        stats_markdown(argv[2], argv[3], argv[4])
    elif argv[1] == "counters":
        counters_markdown(argv[4:], argv[2], argv[3])
    elif argv[1] == "mem-counters":
        memory_counters_markdown(argv[4:], argv[2], argv[3])
    elif argv[1] == "step-counters":
        rec = kernel_busy(argv[6:], argv[3])
        rec.update(kernel=argv[3], workload=argv[4], record=argv[5], source_sha256=source_sha())
        with open(argv[2], "w") as f:
            json.dump(rec, f, indent=1)
    elif argv[1] == "traffic":
        rec = traffic_record(argv[2], argv[3], argv[5], argv[6], int(argv[7]), argv[8], argv[9])
        with open(argv[4], "w") as f:
            json.dump(rec, f, indent=1)
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
