"""Host-side check of the rocprofv3 CSV summariser: kernel names map to the
short names bench.py uses, and counter values are scaled by the calibration
copy's known size."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(f'"{h}"' for h in header) + "\n")
        for r in rows:
            f.write(",".join(f'"{x}"' for x in r) + "\n")


def test_trace_and_traffic(tmp_path):
    d = tmp_path
    _write(str(d / "tr" / "t_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [["void swattn::bwd_dkdv_kernel<128>(int)", 1000, 801000],
            ["void swattn::bwd_dkdv_kernel<128>(int)", 2000, 1002000],
            ["void swattn::attn_fwd_kernel<128>(int)", 0, 300000]])
    out = d / "k.txt"
    subprocess.run([sys.executable, "-m", "sliding_window_causal_qk_amd.rocprof_summary", "trace",
                    "--dir", str(d / "tr"), "--command", "cmd", "--out", str(out)],
                   cwd=ROOT, check=True, capture_output=True)
    txt = out.read_text()
    line = [l for l in txt.splitlines() if l.startswith("bwd_dkdv")][0].split()
    assert line[1] == "2" and float(line[2]) == 900.0
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    neg = "void at::native::vectorized_elementwise_kernel<4, neg_kernel>(int)"
    dq = "void swattn::bwd_dq_kernel<128>(int)"
    _write(str(d / "f" / "p_counter_collection.csv"), hdr,
           [[1, neg, "FETCH_SIZE", 512], [2, dq, "FETCH_SIZE", 100], [3, dq, "FETCH_SIZE", 300]])
    _write(str(d / "w" / "p_counter_collection.csv"), hdr,
           [[1, neg, "WRITE_SIZE", 1024], [2, dq, "WRITE_SIZE", 10], [3, dq, "WRITE_SIZE", 30]])
    subprocess.run([sys.executable, "-m", "sliding_window_causal_qk_amd.rocprof_summary", "traffic",
                    "--fetch", str(d / "f"), "--write", str(d / "w"), "--copy-mib", "1", "--workload", "tiny",
                    "--command-fetch", "a", "--command-write", "b",
                    "--out-json", str(d / "t.json"), "--out-text", str(d / "t.txt")],
                   cwd=ROOT, check=True, capture_output=True)
    rec = json.load(open(d / "t.json"))
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["workload"] == "tiny"
    k = rec["kernels"]["bwd_dq"]
    assert k["launches"] == 2
    assert k["fetch_bytes_per_launch"] == 200 * 1024 * 2.0
    assert k["write_bytes_per_launch"] == 20 * 1024
    assert k["bytes_per_launch"] == k["fetch_bytes_per_launch"] + k["write_bytes_per_launch"]


def test_mfma_counters(tmp_path):
    """Executed FLOPs are MOPS x 512 per dispatch; the busy fraction divides
    the SIMDs' summed MFMA-busy cycles by the per-XCD active cycles (the
    aggregated GRBM_GUI_ACTIVE / 8) times the 1024 SIMDs."""
    d = tmp_path
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    k = "void swattn::bwd_dkdv_kernel<128, false, false>(int)"
    rows = []
    for disp, mops in ((5, 1000), (6, 3000)):
        rows += [[disp, k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops],
                 [disp, k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 50],
                 [disp, k, "GRBM_GUI_ACTIVE", 8 * 200]]
    _write(str(d / "m" / "p_counter_collection.csv"), hdr, rows)
    subprocess.run([sys.executable, "-m", "sliding_window_causal_qk_amd.rocprof_summary", "mfma",
                    "--dir", str(d / "m"), "--workload", "tiny", "--command", "c",
                    "--out-json", str(d / "m.json"), "--out-text", str(d / "m.txt")],
                   cwd=ROOT, check=True, capture_output=True)
    rec = json.load(open(d / "m.json"))
    assert rec["workload"] == "tiny"
    r = rec["kernels"]["bwd_dkdv"]
    assert r["launches"] == 2
    assert r["executed_flops_per_launch"] == 2000 * 512
    assert abs(r["mfma_busy"] - 0.25) < 1e-12
