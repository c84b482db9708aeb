"""Per-kernel summary of rocprofv3 counter runs (``--pmc ... --output-format
csv``), for reading where a kernel's time goes.

    python -m sparse_mixture_experts_top2_amd.counters [--cus 256] [--match REGEX] \\
        run1_counter_collection.csv [run2_counter_collection.csv ...]

Every CSV is one counter pass of the same program; rows are grouped by
kernel name and each counter is averaged over that kernel's dispatches.
Derived columns, where their counters were collected:

* clock (GHz): GRBM_GUI_ACTIVE / 8 (the counter sums the 8 XCDs) over the
  dispatch's duration;
* MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES over the cycles of every SIMD
  (GRBM_GUI_ACTIVE / 8 x CUs x 4), i.e. the matrix cores' duty cycle at the
  clock they ran at;
* LDS conflict: SQ_LDS_BANK_CONFLICT per SQ_ACTIVE_INST_LDS cycle;
* L2 hit: TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum);
* FETCH_SIZE and WRITE_SIZE as read (KiB per dispatch).
"""
from __future__ import annotations

import argparse
import collections
import csv
import re
import sys


def short_name(name: str) -> str:
    name = name.replace("void ", "").replace("moe::(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name).strip()


def load(paths):
    per = collections.defaultdict(dict)          # (kernel, dispatch) -> counter -> value
    meta = {}
    for p in paths:
        with open(p, newline="") as fh:
            for r in csv.DictReader(fh):
                key = (short_name(r["Kernel_Name"]), p, int(r["Dispatch_Id"]))
                per[key][r["Counter_Name"]] = float(r["Counter_Value"])
                per[key]["_dur_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                meta[key[0]] = (r.get("VGPR_Count"), r.get("Accum_VGPR_Count"),
                                r.get("LDS_Block_Size"), r.get("Scratch_Size"))
    return per, meta


def summarize(paths, cus=256, match=None):
    per, meta = load(paths)
    by_kernel = collections.defaultdict(lambda: collections.defaultdict(list))
    for (k, _, _), cs in per.items():
        if match and not re.search(match, k):
            continue
        for c, v in cs.items():
            by_kernel[k][c].append(v)
    rows = []
    for k, cs in by_kernel.items():
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        n = max(len(v) for c, v in cs.items() if c != "_dur_ns")
        row = {"kernel": k, "dispatches": n, "avg_us": mean["_dur_ns"] / 1e3}
        gui = mean.get("GRBM_GUI_ACTIVE")
        if gui:
            row["clock_ghz"] = gui / 8 / mean["_dur_ns"]
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                row["mfma_busy"] = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui / 8 * cus * 4)
        if mean.get("SQ_ACTIVE_INST_LDS"):
            row["lds_conflict"] = mean.get("SQ_LDS_BANK_CONFLICT", 0.0) / mean["SQ_ACTIVE_INST_LDS"]
        if "TCC_HIT_sum" in mean and "TCC_MISS_sum" in mean:
            tot = mean["TCC_HIT_sum"] + mean["TCC_MISS_sum"]
            row["l2_hit"] = mean["TCC_HIT_sum"] / tot if tot else None
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in mean:
                row[c] = mean[c]
        v = meta.get(k)
        if v:
            row["vgpr/agpr/lds/scratch"] = "/".join(str(x) for x in v)
        rows.append(row)
    rows.sort(key=lambda r: -r["avg_us"] * r["dispatches"])
    return rows


def markdown(rows) -> str:
    cols = ["kernel", "dispatches", "avg_us", "clock_ghz", "mfma_busy", "lds_conflict", "l2_hit",
            "FETCH_SIZE", "WRITE_SIZE", "vgpr/agpr/lds/scratch"]
    cols = [c for c in cols if any(c in r for r in rows)]
    out = ["| " + " | ".join(cols) + " |", "|" + "---|" * len(cols)]
    for r in rows:
        cells = []
        for c in cols:
            v = r.get(c)
            if v is None:
                cells.append("")
            elif isinstance(v, float):
                cells.append(f"{v:.3f}" if v < 100 else f"{v:.0f}")
            else:
                cells.append(f"`{v}`" if c == "kernel" else str(v))
        out.append("| " + " | ".join(cells) + " |")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("csv", nargs="+")
    ap.add_argument("--cus", type=int, default=256)
    ap.add_argument("--match", default=None, help="keep kernels whose name matches")
    a = ap.parse_args(argv)
    print(markdown(summarize(a.csv, a.cus, a.match)))


if __name__ == "__main__":
    sys.exit(main())
