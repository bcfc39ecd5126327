"""Summaries of rocprofv3 CSV output as Markdown tables (for profiles/).

    python -m learned_sparse_kv_amd.profsum stats <kernel_stats.csv>
    python -m learned_sparse_kv_amd.profsum pmc [--trace <kernel_stats.csv>] [--kernels REGEX]
                                                <counter_collection.csv> [<more.csv> ...]
    python -m learned_sparse_kv_amd.profsum traffic --workload NAME --fetch <csv> --write <csv>
                                                    [--json profiles/traffic.json]

`stats` prints the kernel-trace statistics (calls, average / min / max
duration, share of GPU time).  `pmc` prints, per kernel, the median over its
dispatches of every collected counter.  Run every dispatch of a kernel at one
shape: the median of mixed shapes describes none of them.

With `--trace` (the kernel statistics of a run with the same arguments and no
counters: counter collection serialises and stretches dispatches, so its own
timestamps and GRBM_GUI_ACTIVE overstate the duration), the table gains the
figures below, each over the kernel's average duration T at the 2.4 GHz
engine clock (f) on 256 CUs / 1,024 SIMDs:

    waves/CU        4 * SQ_WAVE_CYCLES / (T f 256)  (SQ_WAVE_CYCLES counts
                    in units of 4 cycles): waves resident per CU on average
    MFMA busy %     SQ_VALU_MFMA_BUSY_CYCLES / (T f 1024) * 100
    VALU busy %     4 * SQ_ACTIVE_INST_VALU / (T f 1024) * 100 (issue cycles
                    of vector instructions per SIMD, 4 per instruction)
    LDS conflict %  SQ_LDS_BANK_CONFLICT / (T f 256) * 100 (cycles a CU's LDS
                    stalls on bank conflicts)
    MFMA / wave     SQ_INSTS_MFMA / SQ_WAVES
    wait %          SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES * 100 (wave time spent
                    waiting for an instruction's operands or memory)

A bf16 GEMM of known size profiled in the same run (bench.py
--mfma-calibration) shows what a matrix-core-bound kernel reads on the same
counters.

`traffic` turns one FETCH_SIZE run and one WRITE_SIZE run (bench.py
--copy-calibration in both) into HBM bytes per launch: each counter's median
per kernel, scaled by what the same counter reads for the 512 MiB device copy
against the bytes it moves.  The figures go into the JSON file under the
workload's name, each with a hash of its kernel's source, so that a reader
(bench.py's roofline.traffic) uses them only while the source is unchanged;
a Markdown table goes to stdout.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import statistics
import sys
from collections import defaultdict

CUS, SIMDS, CLK = 256, 1024, 2.4e9
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
COPY_BYTES = 512 << 20  # bench.py --copy-calibration

# the source files each kernel is built from
KERNEL_SOURCE = {"k_refine": ["refine_topk.hip"], "k_topk": ["refine_topk.hip"],
                 "k_refine_mfma": ["refine_band.hip"], "k_band_fine": ["refine_band.hip"],
                 "k_key_norm2": ["refine_band.hip"], "k_resolve_sel": ["refine_band.hip"],
                 "k_band_list": ["refine_band.hip"], "k_topk_band": ["refine_band.hip"],
                 "k_attn_mla": ["attn_decode.hip"], "k_attn_f32": ["attn_decode.hip"],
                 "k_attn_merge": ["attn_decode.hip"], "k_score": ["score_select.hip"],
                 "k_select": ["score_select.hip"], "k_fuse_query": ["score_select.hip"],
                 "k_gather": ["gather.hip"], "k_score_sig_mfma": ["score_sigmoid.hip"]}


def source_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def base_name(kernel: str) -> str | None:
    m = re.search(r"\b(k_[a-z0-9_]+)", kernel)
    return m.group(1) if m else None


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


def _durations(path: str) -> dict:
    """Average duration (s) per shortened kernel name from kernel_stats.csv."""
    return {_short(r["Name"]): float(r["AverageNs"]) * 1e-9 for r in csv.DictReader(open(path))}


def derived(m: dict, t: float) -> dict:
    """The figures the module docstring defines, from counter medians m and
    the kernel's duration t (s)."""
    cyc = t * CLK
    d = {"avg µs": t * 1e6}
    if "SQ_WAVE_CYCLES" in m:
        d["waves/CU"] = 4 * m["SQ_WAVE_CYCLES"] / (cyc * CUS)
    if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
        d["MFMA busy %"] = 100 * m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS)
    if "SQ_ACTIVE_INST_VALU" in m:
        d["VALU busy %"] = 100 * 4 * m["SQ_ACTIVE_INST_VALU"] / (cyc * SIMDS)
    if "SQ_LDS_BANK_CONFLICT" in m:
        d["LDS conflict %"] = 100 * m["SQ_LDS_BANK_CONFLICT"] / (cyc * CUS)
    if "SQ_INSTS_MFMA" in m and m.get("SQ_WAVES"):
        d["MFMA / wave"] = m["SQ_INSTS_MFMA"] / m["SQ_WAVES"]
    if "SQ_WAIT_INST_ANY" in m and m.get("SQ_WAVE_CYCLES"):
        d["wait %"] = 100 * m["SQ_WAIT_INST_ANY"] / m["SQ_WAVE_CYCLES"]
    return d


def pmc(paths, trace: str | None = None, kernels: str | None = None) -> str:
    # per (kernel, counter): values over dispatches
    vals = defaultdict(lambda: defaultdict(list))
    meta = {}
    pick = re.compile(kernels) if kernels else None
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = _short(r["Kernel_Name"])
            if pick and not pick.search(r["Kernel_Name"]):
                continue
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            meta.setdefault(k, (r.get("VGPR_Count", ""), r.get("Accum_VGPR_Count", ""),
                                r.get("LDS_Block_Size", r.get("LDS_Size", "")),
                                r.get("Workgroup_Size", "")))
    counters = sorted({c for k in vals for c in vals[k]})
    med = {k: {c: statistics.median(v) for c, v in d.items()} for k, d in vals.items()}
    order = sorted(med, key=lambda k: -max(len(v) for v in vals[k].values()))
    out = []
    head = ["kernel", "dispatches", "VGPR", "AGPR", "LDS B", "WG"] + counters
    out.append("| " + " | ".join(head) + " |")
    out.append("|" + "---|" * len(head))
    for k in order:
        n = max(len(v) for v in vals[k].values())
        row = [f"`{k}`", str(n), *meta[k]] + [f"{med[k].get(c, float('nan')):.0f}" for c in counters]
        out.append("| " + " | ".join(row) + " |")
    if trace:
        dur = _durations(trace)
        der = [(k, derived(med[k], dur[k])) for k in order if k in dur]
        if der:
            names = list(dict.fromkeys(x for _, d in der for x in d))
            out.append("")
            out.append("| kernel | " + " | ".join(names) + " |")
            out.append("|" + "---|" * (len(names) + 1))
            for k, d in der:
                out.append(f"| `{k}` | " + " | ".join(f"{d[x]:.1f}" if x in d else "" for x in names) + " |")
    return "\n".join(out)


def _medians(path: str, counter: str) -> tuple[dict, dict]:
    """Median of the counter per kernel base name, and the launch counts."""
    v = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"].strip()
        key = "__copy" if "copyBuffer" in name else base_name(name)
        if key:
            v[key].append(float(r["Counter_Value"]))
    # the calibration copy is the largest device copy of the run; the
    # kernels take the median over their launches
    med = {k: (max(x) if k == "__copy" else statistics.median(x)) for k, x in v.items()}
    return med, {k: len(x) for k, x in v.items()}


def traffic(workload: str, fetch_csv: str, write_csv: str, json_path: str | None) -> str:
    fm, fn = _medians(fetch_csv, "FETCH_SIZE")
    wm, _ = _medians(write_csv, "WRITE_SIZE")
    if "__copy" not in fm or "__copy" not in wm:
        raise SystemExit("no device copy in the runs: pass --copy-calibration to bench.py")
    kib = COPY_BYTES / 1024
    fs, ws = kib / fm["__copy"], kib / wm["__copy"]
    entry = {}
    for k in sorted(set(fm) & set(wm) - {"__copy"}, key=lambda k: -fm[k]):
        if k not in KERNEL_SOURCE:
            continue
        fb, wb = int(fm[k] * 1024 * fs), int(wm[k] * 1024 * ws)
        entry[k] = {"source_hash": source_hash(KERNEL_SOURCE[k]), "fetch_bytes_per_launch": fb,
                    "write_bytes_per_launch": wb, "bytes_per_launch": fb + wb,
                    "fetch_kib_raw_median": fm[k], "write_kib_raw_median": wm[k], "launches": fn[k]}
    if json_path:
        t = json.load(open(json_path)) if os.path.exists(json_path) else {}
        t[workload] = entry
        t["_calibration"] = {"copy_bytes": COPY_BYTES, "fetch_kib_raw": fm["__copy"],
                             "write_kib_raw": wm["__copy"], "fetch_scale": round(fs, 4),
                             "write_scale": round(ws, 4)}
        with open(json_path, "w") as f:
            json.dump(t, f, indent=1)
            f.write("\n")
    out = [f"Calibration: the {COPY_BYTES >> 20} MiB device copy reads {fm['__copy']:.0f} KiB on FETCH_SIZE "
           f"and {wm['__copy']:.0f} KiB on WRITE_SIZE per dispatch against {kib:.0f} KiB moved each way: "
           f"FETCH_SIZE is scaled by {fs:.3f}, WRITE_SIZE by {ws:.3f}.", "",
           "| kernel | launches | FETCH_SIZE KiB (raw median) | WRITE_SIZE KiB (raw median) | "
           "read MB per launch (scaled) | written MB per launch (scaled) |", "|---|---|---|---|---|---|"]
    for k, e in entry.items():
        out.append(f"| `{k}` | {e['launches']} | {e['fetch_kib_raw_median']:.1f} | {e['write_kib_raw_median']:.1f} | "
                   f"{e['fetch_bytes_per_launch'] / 1e6:.2f} | {e['write_bytes_per_launch'] / 1e6:.2f} |")
    return "\n".join(out)


def main(argv) -> int:
    if len(argv) < 2 or argv[0] not in ("stats", "pmc", "traffic"):
        print(__doc__)
        return 2
    if argv[0] == "stats":
        print(stats(argv[1]))
        return 0
    opts, files = {}, []
    it = iter(argv[1:])
    for a in it:
        if a.startswith("--"):
            opts[a[2:]] = next(it)
        else:
            files.append(a)
    if argv[0] == "traffic":
        print(traffic(opts["workload"], opts["fetch"], opts["write"], opts.get("json")))
    else:
        print(pmc(files, opts.get("trace"), opts.get("kernels")))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
