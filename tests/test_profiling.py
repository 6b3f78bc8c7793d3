"""Host logic of the profile summaries (linear_attention_recurrence_delta_amd/
profiling.py) on small synthetic rocprofv3 CSV files: kernel-name labels,
copy-calibrated traffic, and the MFMA counter table. CPU only."""
import csv
import json

from linear_attention_recurrence_delta_amd import profiling as P

SCAN = "_ZN3gdn12_GLOBAL__N_111gdn_k3_scanIDF16bLi128ELi64ELb0ELb0ELb0EEEvNS_11PrefillArgsE"
SCAN_SAVE = "_ZN3gdn12_GLOBAL__N_111gdn_k3_scanIDF16bLi128ELi64ELb0ELb1ELb0EEEvNS_11PrefillArgsE"
SCAN_WIN = "_ZN3gdn12_GLOBAL__N_111gdn_k3_scanIDF16bLi128ELi64ELb0ELb0ELb1EEEvNS_11PrefillArgsE"
K2_BWD = "_ZN3gdn12_GLOBAL__N_116gdn_k2_inverse_wIDF16bLi128ELi64ELb0ELb0ELb1ELb0EEEvNS_11PrefillArgsE"
K2_PREP = ("void gdn::(anonymous namespace)::gdn_k2_inverse_w<__hip_bfloat16, 128, 64, true, false, false, "
           "false>(gdn::PrefillArgs)")
K2_WIN = ("void gdn::(anonymous namespace)::gdn_k2_inverse_w<__hip_bfloat16, 128, 64, false, false, false, "
          "true>(gdn::PrefillArgs)")
COPY = "__amd_rocclr_copyBuffer"


def write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, counter, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_short_names_label_true_switches():
    assert P.short_name(SCAN) == "gdn_k3_scan"
    assert P.short_name(SCAN_SAVE) == "gdn_k3_scan [save]"
    assert P.short_name(K2_BWD) == "gdn_k2_inverse_w [bwd]"
    assert P.short_name(K2_PREP) == "gdn_k2_inverse_w [prep]"
    # the launches of a window beside the scan
    assert P.short_name(SCAN_WIN) == "gdn_k3_scan [window]"
    assert P.short_name(K2_WIN) == "gdn_k2_inverse_w [window]"
    assert P.source_of("gdn_k2_inverse_w [bwd]") == "gdn_prefill.hip"
    assert P.source_of(COPY) is None


def test_traffic_scales_by_the_copy_and_takes_medians(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cfetch, cwrite = tmp_path / "cf.csv", tmp_path / "cw.csv"
    # the scan's three dispatches: median fetch 100 KiB, write 40 KiB
    write_counters(fetch, [(SCAN, "FETCH_SIZE", 90), (SCAN, "FETCH_SIZE", 100), (SCAN, "FETCH_SIZE", 500)])
    write_counters(write, [(SCAN, "WRITE_SIZE", 40), (SCAN, "WRITE_SIZE", 40), (SCAN, "WRITE_SIZE", 41)])
    # a 1 MiB copy whose FETCH_SIZE reads half and WRITE_SIZE all of it
    write_counters(cfetch, [(COPY, "FETCH_SIZE", 512)])
    write_counters(cwrite, [(COPY, "WRITE_SIZE", 1024)])
    out = P.traffic(str(fetch), str(write), str(cfetch), str(cwrite), 1 << 20)
    assert out["_calibration"]["fetch_scale"] == 2.0 and out["_calibration"]["write_scale"] == 1.0
    rec = out["gdn_k3_scan"]
    assert rec["fetch_bytes"] == 100 * 1024 * 2 and rec["write_bytes"] == 40 * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["source"] == "gdn_prefill.hip" and len(rec["source_sha256"]) == 64


def test_mfma_table_rates(tmp_path):
    counters, stats, bench = tmp_path / "c.csv", tmp_path / "s.csv", tmp_path / "b.json"
    write_counters(counters, [(SCAN, "MfmaUtil", 11.5), (SCAN, "MfmaFlopsBF16", 2.5e11)])
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs",
                                          "Percentage"])
        w.writeheader()
        w.writerow({"Name": SCAN, "Calls": 2, "TotalDurationNs": 2.0e6, "AverageNs": 1.0e6, "MinNs": 1.0e6,
                    "MaxNs": 1.0e6, "Percentage": 100})
    # bench: 0.1 of bf16 peak over 1 ms is 250 GFLOP of algorithmic work
    bench.write_text(json.dumps({"kernels": {"gdn_k3_scan": {"ms": 1.0, "mfma_frac": 0.1}}}) + "\n")
    table = P.mfma_table(str(counters), str(stats), str(bench))
    row = [r for r in table.splitlines() if r.startswith("| gdn_k3_scan")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    # executed 250 G flops over a 1000 us mean: 250 TFLOP/s, 0.1 of peak; algorithmic / executed 1.00
    assert cells[1] == "11.5" and cells[2] == "250.0" and cells[3] == "1000.0"
    assert cells[4] == "250.0" and cells[5] == "0.1000" and cells[6] == "250.0" and cells[7] == "1.00"
