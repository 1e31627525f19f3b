"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m hybrid_prefill_decode_paged_amd.profiling stats  <kernel_stats.csv> <out.md> <command...>
    python -m hybrid_prefill_decode_paged_amd.profiling traffic <copy_fetch_dir> <copy_write_dir> \
        <fetch_dir> <write_dir> <kernel-substring> <out.json> <command...>
    python -m hybrid_prefill_decode_paged_amd.profiling pmc <out.md> <title> <command> <dir>...

pmc: per-kernel mean of every counter over its dispatches, for each counter-collection
directory given (one rocprofv3 --pmc pass each), as one markdown table.

Traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernel, each scaled by the ratio of
the true byte count to what the same counter reads for a plain 1 GiB device copy
(``python bench.py --calibrate-copy``: 1 GiB read + 1 GiB written per dispatch).  The record
carries the SHA-256 of the kernel sources so that bench.py reports it only while the kernels
are unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/pod_kernels.hip", "csrc/pod_internal.h", "csrc/plan.cpp", "csrc/pod_api.cpp")
COPY_BYTES = 1 << 30
MI355X_XCDS = 8
MI355X_SIMDS = 256 * 4


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _counter_csv(d: str) -> str:
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    return files[0]


def per_dispatch(d: str, kernel_substr: str, counter: str):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(_counter_csv(d)))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise ValueError(f"{counter} for '{kernel_substr}' not found in {d}")
    return statistics.mean(vals), len(vals)


def traffic_record(copy_fetch, copy_write, fetch, write, kernel_substr, command):
    cf, _ = per_dispatch(copy_fetch, "copyBuffer", "FETCH_SIZE")
    cw, _ = per_dispatch(copy_write, "copyBuffer", "WRITE_SIZE")
    f, nf = per_dispatch(fetch, kernel_substr, "FETCH_SIZE")
    w, nw = per_dispatch(write, kernel_substr, "WRITE_SIZE")
    fs, ws = (COPY_BYTES / 1024) / cf, (COPY_BYTES / 1024) / cw
    return {
        "kernel": kernel_substr,
        "fetch_kib_per_dispatch": round(f, 1), "write_kib_per_dispatch": round(w, 1),
        "dispatches": [nf, nw],
        "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
        "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
        "traffic_bytes_per_dispatch": int(round((f * fs + w * ws) * 1024)),
        "kernel_source_sha256": kernel_source_hash(),
        "command": command,
    }


def stats_summary(path: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 kernel statistics", "", f"Command: `{command}`", "",
           "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")
        short = name.split("(")[0][:90]
        out.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out) + "\n"


def pmc_summary(dirs, title: str, command: str) -> str:
    rows = {}
    for d in dirs:
        for r in csv.DictReader(open(_counter_csv(d))):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
            if "pod_" not in name:
                continue
            rows.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    counters = sorted({c for v in rows.values() for c in v})
    busy = "SQ_VALU_MFMA_BUSY_CYCLES" in counters and "GRBM_GUI_ACTIVE" in counters
    extra = ["MFMA busy"] if busy else []
    out = [f"# {title}", "", f"Command: `{command}`", "",
           "Per-dispatch mean of each counter (summed over the device by rocprofv3), dispatches in brackets."]
    if busy:
        out += ["MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x SIMDs): the share of the "
                f"kernel's span in which a SIMD's matrix core is busy, averaged over the {MI355X_SIMDS} SIMDs "
                f"(GRBM_GUI_ACTIVE is summed over the {MI355X_XCDS} XCDs)."]
    out += ["", "| kernel | " + " | ".join(counters + extra) + " |", "|---" * (len(counters) + len(extra) + 1) + "|"]
    for name, d in rows.items():
        cells = [f"{statistics.mean(d[c]):.4g} ({len(d[c])})" if c in d else "" for c in counters]
        if busy:
            span = statistics.mean(d["GRBM_GUI_ACTIVE"]) / MI355X_XCDS * MI355X_SIMDS if "GRBM_GUI_ACTIVE" in d else 0
            mf = statistics.mean(d["SQ_VALU_MFMA_BUSY_CYCLES"]) if "SQ_VALU_MFMA_BUSY_CYCLES" in d else None
            cells.append(f"{100 * mf / span:.1f}%" if span and mf is not None else "")
        out.append(f"| {name[:70]} | " + " | ".join(cells) + " |")
    return "\n".join(out) + "\n"


def main(argv):
    if argv[0] == "stats":
        open(argv[2], "w").write(stats_summary(argv[1], " ".join(argv[3:])))
    elif argv[0] == "pmc":
        open(argv[1], "w").write(pmc_summary(argv[4:], argv[2], argv[3]))
    elif argv[0] == "traffic":
        rec = traffic_record(*argv[1:6], " ".join(argv[7:]))
        json.dump(rec, open(argv[6], "w"), indent=1)
        print(json.dumps(rec))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
