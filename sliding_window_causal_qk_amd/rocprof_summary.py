"""Turn rocprofv3 CSV output of a bench.py run into the short text summaries
kept with the library, and into the per-launch HBM traffic table that
bench.py reports beside its roofline.

    # kernel durations: rocprofv3 --kernel-trace --stats -f csv -d DIR -- python3 bench.py ...
    python -m sliding_window_causal_qk_amd.rocprof_summary trace --dir DIR --command "..." --out FILE

    # HBM bytes: two counter runs of bench.py --copy-calibration-mib M (FETCH_SIZE, then WRITE_SIZE)
    python -m sliding_window_causal_qk_amd.rocprof_summary traffic --fetch DIR1 --write DIR2 \\
        --copy-mib M --command-fetch "..." --command-write "..." --out-json J --out-text FILE

    # executed MFMA work: one counter run of bench.py with
    #   --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
    python -m sliding_window_causal_qk_amd.rocprof_summary mfma --dir DIR --workload W \
        --command "..." --out-json J --out-text FILE

FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch.  Each is scaled by the
ratio of the known byte count of the calibration copy (torch.neg over M MiB of
fp32: M MiB read, M MiB written) to what the same counter reads for it.

SQ_INSTS_VALU_MFMA_MOPS_BF16 counts bf16 MFMA operations in units of 512, so
x 512 is the FLOPs the matrix cores executed (masked blocks and recomputation
included).  The MFMA busy fraction follows rocprofv3's own MfmaUtil metric,
SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs / (the per-XCD maximum of
GRBM_GUI_ACTIVE x SIMDs); rocprofv3 aggregates GRBM_GUI_ACTIVE over the XCDs
by summing, so its per-XCD value is taken as the sum / XCDS.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# kernel symbol fragment -> short name used by bench.py
# (the key pre-pass is one kernel in both passes: its forward and backward
# launches share one name and one average)
SHORT = (("key_prep_kernel", "key_prep"), ("attn_fwd_kernel", "attn_fwd"), ("bwd_dkdv_kernel", "bwd_dkdv"),
         ("bwd_dkdv_split_kernel", "bwd_dkdv"),
         ("bwd_dq_kernel", "bwd_dq"), ("ve_gate_bwd_kernel", "ve_gate_bwd"), ("ve_gate_dw_kernel", "ve_gate_dw"))


def short_name(kernel: str) -> str | None:
    for frag, name in SHORT:
        if frag in kernel:
            return name
    return None


def kernel_sources_sha() -> str:
    """Same digest as bench.py: every file of the kernel sources, by name."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sliding_window_causal_qk_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        sys.exit(f"no *{suffix} under {d}")
    return hits[-1]


def _rows(path: str):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _col(row: dict, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in columns {list(row)}")


def trace(args):
    rows = _rows(_find(args.dir, "kernel_trace.csv"))
    rows.sort(key=lambda r: int(_col(r, "Start_Timestamp", "Start-Timestamp")))
    per = {}
    for r in rows:
        name = _col(r, "Kernel_Name", "Kernel-Name", "Name")
        dur = (int(_col(r, "End_Timestamp", "End-Timestamp")) - int(_col(r, "Start_Timestamp", "Start-Timestamp"))) / 1e3
        per.setdefault(name, []).append(dur)
    if args.skip_first:   # drop each kernel's first launches (the warm-up step)
        per = {k: v[args.skip_first:] for k, v in per.items() if len(v) > args.skip_first}
    total = sum(sum(v) for v in per.values())
    lines = [f"# rocprofv3 kernel trace: {args.title}", "",
             "Command (from the repository root):", "", "    " + args.command, "",
             f"Launches counted: all but the first {args.skip_first} of each kernel." if args.skip_first else
             "Launches counted: all.", "",
             f"{'kernel':<12} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'total_ms':>9} {'pct':>6}  symbol"]
    for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{(short_name(name) or '-'):<12} {len(d):>6} {statistics.fmean(d):>9.2f} {min(d):>9.2f} "
                     f"{max(d):>9.2f} {sum(d) / 1e3:>9.3f} {100 * sum(d) / total:>6.2f}  {name[:90]}")
    lines += ["", f"kernel sources sha: {kernel_sources_sha()}"]
    txt = "\n".join(lines) + "\n"
    if args.out:
        open(args.out, "w").write(txt)
    print(txt)


def _counter_means(d: str, counter: str):
    rows = _rows(_find(d, "counter_collection.csv"))
    per = {}
    for r in rows:
        if _col(r, "Counter_Name", "Counter-Name") != counter:
            continue
        name = _col(r, "Kernel_Name", "Kernel-Name")
        per.setdefault(name, []).append(float(_col(r, "Counter_Value", "Counter-Value")))
    return {k: statistics.fmean(v) for k, v in per.items()}, {k: len(v) for k, v in per.items()}


XCDS, SIMDS = 8, 256 * 4   # MI355X: 8 XCDs, 256 CUs of 4 SIMDs


def mfma(args):
    rows = _rows(_find(args.dir, "counter_collection.csv"))
    per = {}
    for r in rows:
        name = short_name(_col(r, "Kernel_Name", "Kernel-Name"))
        if name is None:
            continue
        key = (name, _col(r, "Dispatch_Id", "Dispatch-Id"))
        d = per.setdefault(key, {})
        d[_col(r, "Counter_Name", "Counter-Name")] = float(_col(r, "Counter_Value", "Counter-Value"))
    agg = {}
    for (name, _), d in per.items():
        a = agg.setdefault(name, {"n": 0, "flops": 0.0, "busy": 0.0, "cycles": 0.0})
        a["n"] += 1
        a["flops"] += d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        a["busy"] += d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        a["cycles"] += d.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
    out = {"sources_sha": kernel_sources_sha(), "workload": args.workload, "command": args.command,
           "kernels": {}}
    lines = [f"# Executed MFMA work per launch from rocprofv3 counters: {args.title}", "",
             "Command (from the repository root):", "", "    " + args.command, "",
             "Executed FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
             f"(GRBM_GUI_ACTIVE / {XCDS} XCDs x {SIMDS} SIMDs), rocprofv3's MfmaUtil.", "",
             f"{'kernel':<10} {'launches':>8} {'exec_GFLOP':>11} {'mfma_busy':>10}"]
    for name, a in sorted(agg.items()):
        n = a["n"]
        fl = a["flops"] / n
        busy = a["busy"] / (a["cycles"] * SIMDS) if a["cycles"] else 0.0
        out["kernels"][name] = {"executed_flops_per_launch": fl, "mfma_busy": busy, "launches": n}
        lines.append(f"{name:<10} {n:>8} {fl / 1e9:>11.1f} {100 * busy:>9.1f}%")
    lines += ["", f"kernel sources sha: {out['sources_sha']}"]
    json.dump(out, open(args.out_json, "w"), indent=1)
    txt = "\n".join(lines) + "\n"
    open(args.out_text, "w").write(txt)
    print(txt)


def traffic(args):
    fetch, nf = _counter_means(args.fetch, "FETCH_SIZE")
    write, nw = _counter_means(args.write, "WRITE_SIZE")
    copy_bytes = args.copy_mib * 1024 * 1024
    cf = [k for k in fetch if "neg" in k]
    cw = [k for k in write if "neg" in k]
    if not cf or not cw:
        sys.exit("calibration copy (torch.neg) not found in the counter output")
    f_fac = copy_bytes / (fetch[cf[0]] * 1024.0)
    w_fac = copy_bytes / (write[cw[0]] * 1024.0)
    out = {"sources_sha": kernel_sources_sha(), "workload": args.workload, "copy_mib": args.copy_mib,
           "fetch_factor": f_fac, "write_factor": w_fac,
           "command_fetch": args.command_fetch, "command_write": args.command_write, "kernels": {}}
    lines = [f"# HBM traffic per launch from rocprofv3 counters: {args.title}", "",
             "Commands (from the repository root):", "", "    " + args.command_fetch, "    " + args.command_write, "",
             f"Calibration: torch.neg over {args.copy_mib} MiB fp32 reads FETCH_SIZE {fetch[cf[0]]:.0f} KiB and "
             f"WRITE_SIZE {write[cw[0]]:.0f} KiB per launch for {copy_bytes // 1024} KiB each; "
             f"scale factors {f_fac:.4f} (fetch), {w_fac:.4f} (write).", "",
             f"{'kernel':<10} {'launches':>8} {'fetch_MB':>10} {'write_MB':>10} {'total_MB':>10}"]
    for k in fetch:
        name = short_name(k)
        if name is None or k not in write:
            continue
        fb, wb = fetch[k] * 1024.0 * f_fac, write[k] * 1024.0 * w_fac
        out["kernels"][name] = {"fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                                "bytes_per_launch": fb + wb, "launches": nf[k]}
        lines.append(f"{name:<10} {nf[k]:>8} {fb / 1e6:>10.1f} {wb / 1e6:>10.1f} {(fb + wb) / 1e6:>10.1f}")
    lines += ["", f"kernel sources sha: {out['sources_sha']}"]
    json.dump(out, open(args.out_json, "w"), indent=1)
    txt = "\n".join(lines) + "\n"
    open(args.out_text, "w").write(txt)
    print(txt)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="")
    t.add_argument("--skip-first", type=int, default=0,
                   help="ignore the first N launches of every kernel (a warm-up step)")
    t.add_argument("--out")
    c = sub.add_parser("traffic")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-mib", type=int, required=True)
    c.add_argument("--workload", required=True, help="the bench.py workload the counter runs measured")
    c.add_argument("--command-fetch", required=True)
    c.add_argument("--command-write", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--out-json", required=True)
    c.add_argument("--out-text", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--dir", required=True)
    m.add_argument("--workload", required=True, help="the bench.py workload the counter run measured")
    m.add_argument("--command", required=True)
    m.add_argument("--title", default="")
    m.add_argument("--out-json", required=True)
    m.add_argument("--out-text", required=True)
    a = ap.parse_args()
    {"trace": trace, "traffic": traffic, "mfma": mfma}[a.mode](a)


if __name__ == "__main__":
    main()
