"""Host logic of the rocprofv3 summariser (no GPU): counter medians per
kernel, the derived figures over a trace duration, and the traffic scaling
against the device copy."""
import csv
import json

from learned_sparse_kv_amd import profsum

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "VGPR_Count",
          "Accum_VGPR_Count", "LDS_Block_Size", "Workgroup_Size"]


def _pmc_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v,
                        "VGPR_Count": 8, "Accum_VGPR_Count": 0, "LDS_Block_Size": 0, "Workgroup_Size": 256})


def test_derived_figures_over_trace_duration(tmp_path):
    k = "void (anonymous namespace)::k_attn_mla<8, 1>(GeomDev)"
    t = 10e-6
    cyc = t * profsum.CLK
    _pmc_csv(tmp_path / "c.csv", [(k, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * 1024),
                                  (k, "SQ_VALU_MFMA_BUSY_CYCLES", 0.1 * cyc * 1024),
                                  (k, "SQ_VALU_MFMA_BUSY_CYCLES", 0.3 * cyc * 1024),
                                  (k, "SQ_WAVE_CYCLES", 8 * cyc * 256 / 4),
                                  (k, "SQ_INSTS_MFMA", 680 * 2048), (k, "SQ_WAVES", 2048)])
    with open(tmp_path / "s.csv", "w") as f:
        f.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        f.write(f'"{k}",3,30000,{t * 1e9},100,9000,11000,1\n')
    md = profsum.pmc([str(tmp_path / "c.csv")], trace=str(tmp_path / "s.csv"))
    last = md.strip().splitlines()[-1]
    cells = [c.strip() for c in last.strip("|").split("|")]
    head = [c.strip() for c in md.strip().splitlines()[-3].strip("|").split("|")]
    d = dict(zip(head, cells))
    assert d["avg µs"] == "10.0"
    assert d["MFMA busy %"] == "30.0"  # the median of the three dispatches
    assert d["waves/CU"] == "8.0"
    assert d["MFMA / wave"] == "680.0"


def test_traffic_scaled_by_copy_and_hashed(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    k = "void (anonymous namespace)::k_attn_mla<8, 1>(GeomDev)"
    _pmc_csv(tmp_path / "f.csv", [(copy, "FETCH_SIZE", 4.0), (copy, "FETCH_SIZE", 262144.0),
                                  (copy, "FETCH_SIZE", 8.0), (k, "FETCH_SIZE", 1000.0),
                                  (k, "FETCH_SIZE", 1200.0), (k, "FETCH_SIZE", 1100.0)])
    _pmc_csv(tmp_path / "w.csv", [(copy, "WRITE_SIZE", 524288.0), (copy, "WRITE_SIZE", 5.0),
                                  (k, "WRITE_SIZE", 10.0)])
    out = tmp_path / "t.json"
    profsum.traffic("wl", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out))
    t = json.load(open(out))
    e = t["wl"]["k_attn_mla"]
    assert e["fetch_bytes_per_launch"] == 1100 * 1024 * 2  # the copy's reads count half
    assert e["write_bytes_per_launch"] == 10 * 1024
    assert e["source_hash"] == profsum.source_hash(profsum.KERNEL_SOURCE["k_attn_mla"])
    assert t["_calibration"]["fetch_scale"] == 2.0
