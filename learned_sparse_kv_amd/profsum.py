"""Summaries of rocprofv3 CSV output as Markdown tables (for profiles/).

    python -m learned_sparse_kv_amd.profsum stats <kernel_stats.csv>
    python -m learned_sparse_kv_amd.profsum pmc <counter_collection.csv> [<more.csv> ...]

`stats` prints the kernel-trace statistics (calls, average / min / max
duration, share of GPU time).  `pmc` prints, per kernel, the median over its
dispatches of every collected counter, and the derived figures that the
counters present allow:

    occupancy %     SQ_WAVE_CYCLES / (GRBM_GUI_ACTIVE * CUs * 32 waves) * 400
                    (resident waves as a share of the CU's maximum; the
                    counter is sampled per SIMD, hence the factor 4)
    MFMA busy %     SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs) * 100
    VALU busy %     SQ_ACTIVE_INST_VALU / (GRBM_GUI_ACTIVE * CUs) * 100
    LDS conflict %  SQ_LDS_BANK_CONFLICT / (GRBM_GUI_ACTIVE * CUs) * 100
    wait %          SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES * 100 (wave cycles spent
                    waiting for an instruction's operands or memory)

(the expressions of rocprofv3's own derived counters OccupancyPercent,
MfmaUtil, VALUBusy and LDSBankConflict; 256 CUs and 1,024 SIMDs on MI355X).
"""
from __future__ import annotations

import csv
import statistics
import sys
from collections import defaultdict

CUS, SIMDS = 256, 1024


def _short(name: str, width: int = 60) -> str:
    name = name.strip()
    return name if len(name) <= width else name[:width]


def stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    out = ["| kernel | calls | avg µs | min µs | max µs | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{100 * float(r['TotalDurationNs']) / tot:.1f} % |")
    return "\n".join(out)


def pmc(paths) -> str:
    # per (kernel, counter): values over dispatches
    vals = defaultdict(lambda: defaultdict(list))
    meta = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = _short(r["Kernel_Name"])
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            meta.setdefault(k, (r.get("VGPR_Count", ""), r.get("Accum_VGPR_Count", ""),
                                r.get("LDS_Block_Size", r.get("LDS_Size", "")),
                                r.get("Workgroup_Size", "")))
    counters = sorted({c for k in vals for c in vals[k]})
    med = {k: {c: statistics.median(v) for c, v in d.items()} for k, d in vals.items()}
    out = []
    head = ["kernel", "dispatches", "VGPR", "AGPR", "LDS B", "WG"] + counters
    out.append("| " + " | ".join(head) + " |")
    out.append("|" + "---|" * len(head))
    for k in sorted(med, key=lambda k: -len(vals[k][counters[0]]) if counters[0] in vals[k] else 0):
        n = max(len(v) for v in vals[k].values())
        row = [f"`{k}`", str(n), *meta[k]] + [f"{med[k].get(c, float('nan')):.0f}" for c in counters]
        out.append("| " + " | ".join(row) + " |")
    der = []
    for k, m in med.items():
        g = m.get("GRBM_GUI_ACTIVE")
        if not g:
            continue
        d = {}
        if "SQ_WAVE_CYCLES" in m:
            d["occupancy %"] = 400 * m["SQ_WAVE_CYCLES"] / (g * CUS * 32)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            d["MFMA busy %"] = 100 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * SIMDS)
        if "SQ_ACTIVE_INST_VALU" in m:
            d["VALU busy %"] = 100 * m["SQ_ACTIVE_INST_VALU"] / (g * CUS)
        if "SQ_LDS_BANK_CONFLICT" in m:
            d["LDS conflict %"] = 100 * m["SQ_LDS_BANK_CONFLICT"] / (g * CUS)
        if "SQ_WAIT_INST_ANY" in m and m.get("SQ_WAVE_CYCLES"):
            d["wait %"] = 100 * m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"]
        if d:
            der.append((k, d))
    if der:
        names = sorted({x for _, d in der for x in d})
        out.append("")
        out.append("| kernel | " + " | ".join(names) + " |")
        out.append("|" + "---|" * (len(names) + 1))
        for k, d in der:
            out.append(f"| `{k}` | " + " | ".join(f"{d[x]:.1f}" if x in d else "" for x in names) + " |")
    return "\n".join(out)


if __name__ == "__main__":
    if len(sys.argv) < 3 or sys.argv[1] not in ("stats", "pmc"):
        print(__doc__)
        sys.exit(2)
    print(stats(sys.argv[2]) if sys.argv[1] == "stats" else pmc(sys.argv[2:]))
