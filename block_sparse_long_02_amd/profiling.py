"""Summaries of rocprofv3 output for the profiles/ folder.

  python -m block_sparse_long_02_amd.profiling stats <kernel_stats.csv> --title T --command C
      -> markdown table of per-kernel call counts and durations
  python -m block_sparse_long_02_amd.profiling traffic --fetch <dir> --write <dir>
         --kernel kv_outer_kernel --copy-bytes N --out <json> --command C
      -> per-launch HBM traffic of a kernel from two --pmc passes (FETCH_SIZE,
         WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
         reads for the blit copy kernel of N bytes in the same run
  python -m block_sparse_long_02_amd.profiling counters --dirs <dir> [<dir> ...]
         --kernels k1,k2 --title T --command C --out <md>
      -> per-dispatch SQ counters of the kernels (summed over the shader
         engines) with instruction mix and MFMA-busy ratios
  python -m block_sparse_long_02_amd.profiling clocks --dir <dir> --kernels k1,k2
         --title T --command C --out <md>
      -> the clock each kernel ran at (GRBM_GUI_ACTIVE per XCD over the
         dispatch's duration) and its MFMA-busy share of those cycles

The traffic file records a hash of the kernel's sources; bench.py reports the
traffic only while the sources still match.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_KERNEL = "__amd_rocclr_copyBuffer"

# sources (and build flags) whose change invalidates measured counters of a kernel
KERNEL_SOURCES = {
    "index_blockmax_prefill_kernel": ["csrc/index_blockmax.hip", "csrc/msa_device.h", "csrc/msa_internal.h",
                                      "build.py"],
    "kv_outer_kernel": ["csrc/sparse_attn.hip", "csrc/msa_device.h", "csrc/msa_internal.h", "csrc/api.hip",
                        "build.py"],
    "query_major_kernel": ["csrc/sparse_attn.hip", "csrc/msa_device.h", "csrc/msa_internal.h", "csrc/api.hip",
                           "build.py"],
    "decode_index_kernel": ["csrc/decode.hip", "csrc/msa_device.h", "csrc/msa_internal.h", "csrc/api.hip",
                            "build.py"],
    "decode_attn_kernel": ["csrc/decode.hip", "csrc/msa_device.h", "csrc/msa_internal.h", "csrc/api.hip",
                           "build.py"],
    "bwd_list_kernel": ["csrc/backward.hip", "csrc/msa_device.h", "csrc/msa_internal.h", "csrc/api.hip",
                        "build.py"],
    "dense_attn_kernel": ["csrc/sparse_attn.hip", "csrc/msa_device.h", "csrc/msa_internal.h", "csrc/api.hip",
                          "build.py"],
    "index_topk_one_pass_kernel": ["csrc/index_blockmax.hip", "csrc/msa_device.h", "csrc/msa_internal.h",
                                   "csrc/api.hip", "build.py"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_stats_md(path: str, title: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", command, "```", "",
           "| kernel | calls | avg ms | total ms | % of kernel time |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| {r['Name'][:80]} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def _counter_rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _per_dispatch(rows, kernel: str, counter: str):
    vals = {}
    for r in rows:
        if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
            key = r.get("Dispatch_Id") or r.get("Correlation_Id")
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def pmc_traffic(fetch_dir: str, write_dir: str, kernel: str, copy_bytes: int) -> dict:
    fr, wr = _counter_rows(fetch_dir), _counter_rows(write_dir)
    f_k, w_k = _per_dispatch(fr, kernel, "FETCH_SIZE"), _per_dispatch(wr, kernel, "WRITE_SIZE")
    f_c, w_c = _per_dispatch(fr, COPY_KERNEL, "FETCH_SIZE"), _per_dispatch(wr, COPY_KERNEL, "WRITE_SIZE")
    if not (f_k and w_k and f_c and w_c):
        raise ValueError("missing dispatches for the kernel or the calibration copy")
    # the largest copy dispatch is the calibration copy of copy_bytes
    fac_f = copy_bytes / (max(f_c) * 1024.0)
    fac_w = copy_bytes / (max(w_c) * 1024.0)
    fetch = sum(f_k) / len(f_k) * 1024.0 * fac_f
    write = sum(w_k) / len(w_k) * 1024.0 * fac_w
    return {"kernel": kernel, "launches": len(f_k), "fetch_bytes_per_launch": fetch,
            "write_bytes_per_launch": write, "traffic_bytes_per_launch": fetch + write,
            "fetch_kib_raw": sum(f_k) / len(f_k), "write_kib_raw": sum(w_k) / len(w_k),
            "copy_factor_fetch": fac_f, "copy_factor_write": fac_w, "copy_bytes": copy_bytes,
            "source_sha256": source_hash(kernel)}


# MI355X: 256 CUs in 32 shader engines, 4 SIMDs per CU
SIMDS_PER_SE = 32
N_SIMDS = 1024


def counters_md(dirs, kernels, title: str, command: str) -> str:
    rows = []
    for d in dirs:
        rows += _counter_rows(d)
    names = sorted({r["Counter_Name"] for r in rows})
    per = {}
    for k in kernels:
        per[k] = {}
        for c in names:
            v = _per_dispatch(rows, k, c)
            if v:
                per[k][c] = sum(v) / len(v)
    out = [f"# {title}", "", "Commands (from the repository root, on one MI355X; one pass per counter set):", "",
           "```", command, "```", "",
           "Values are per dispatch, averaged over the dispatches of the kernel, each summed over the shader "
           "engines (SQ counters).", "",
           "| counter | " + " | ".join(kernels) + " |", "|---|" + "---:|" * len(kernels)]
    for c in names:
        out.append(f"| {c} | " + " | ".join(f"{per[k].get(c, float('nan')):.4g}" for k in kernels) + " |")

    def ratio(k, a, b, scale=1.0):
        x, y = per[k].get(a), per[k].get(b)
        return f"{x / (y * scale):.3f}" if x is not None and y else "n/a"
    out += ["", "Derived:", "", "| ratio | " + " | ".join(kernels) + " |", "|---|" + "---:|" * len(kernels),
            "| VALU instructions per MFMA instruction | " +
            " | ".join(ratio(k, "SQ_INSTS_VALU", "SQ_INSTS_MFMA") for k in kernels) + " |",
            "| LDS instructions per MFMA instruction | " +
            " | ".join(ratio(k, "SQ_INSTS_LDS", "SQ_INSTS_MFMA") for k in kernels) + " |",
            f"| MFMA busy / (SQ busy x {SIMDS_PER_SE} SIMDs per engine) | " +
            " | ".join(ratio(k, "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", SIMDS_PER_SE) for k in kernels) + " |",
            "| waves' cycles waiting on any instruction / wave cycles | " +
            " | ".join(ratio(k, "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES") for k in kernels) + " |"]
    return "\n".join(out) + "\n"


N_XCDS = 8


def _dispatch_clocks(rows, kernel: str):
    """Per dispatch of `kernel`: (seconds, GRBM_GUI_ACTIVE per XCD, MFMA busy cycles per SIMD)."""
    per = {}
    for r in rows:
        if kernel not in r["Kernel_Name"]:
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        d = per.setdefault(key, {"dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = []
    for d in per.values():
        if d["dur"] > 0 and "GRBM_GUI_ACTIVE" in d:
            out.append((d["dur"], d["GRBM_GUI_ACTIVE"] / N_XCDS, d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / N_SIMDS))
    return out


def clocks_md(d: str, kernels, title: str, command: str) -> str:
    rows = _counter_rows(d)
    out = [f"# {title}", "", "Command (from the repository root, on one MI355X):", "", "```", command, "```", "",
           f"Clock = GRBM_GUI_ACTIVE / {N_XCDS} XCDs / dispatch duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
           f"{N_SIMDS} SIMDs / those cycles; MFMA peak at that clock = 1024 flop per SIMD per cycle x {N_SIMDS} "
           "SIMDs. Averages over the kernel's dispatches.", "",
           "| kernel | dispatches | avg ms | clock GHz | MFMA busy | bf16 MFMA peak at that clock, PFLOP/s |",
           "|---|---:|---:|---:|---:|---:|"]
    for k in kernels:
        v = _dispatch_clocks(rows, k)
        if not v:
            continue
        dur = sum(x[0] for x in v) / len(v)
        clk = sum(x[1] / x[0] for x in v) / len(v)
        busy = sum(x[2] / x[1] for x in v) / len(v)
        out.append(f"| {k} | {len(v)} | {dur * 1e3:.3f} | {clk / 1e9:.3f} | {busy:.3f} | "
                   f"{clk * 1024 * N_SIMDS / 1e15:.3f} |")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s1 = sub.add_parser("stats")
    s1.add_argument("csv")
    s1.add_argument("--title", required=True)
    s1.add_argument("--command", required=True)
    s1.add_argument("--out")
    s2 = sub.add_parser("traffic")
    s2.add_argument("--fetch", required=True)
    s2.add_argument("--write", required=True)
    s2.add_argument("--kernel", required=True)
    s2.add_argument("--copy-bytes", type=int, required=True)
    s2.add_argument("--command", required=True)
    s2.add_argument("--out", required=True)
    s3 = sub.add_parser("counters")
    s3.add_argument("--dirs", nargs="+", required=True)
    s3.add_argument("--kernels", required=True)
    s3.add_argument("--title", required=True)
    s3.add_argument("--command", required=True)
    s3.add_argument("--out")
    s4 = sub.add_parser("clocks")
    s4.add_argument("--dir", required=True)
    s4.add_argument("--kernels", required=True)
    s4.add_argument("--title", required=True)
    s4.add_argument("--command", required=True)
    s4.add_argument("--out")
    a = ap.parse_args()
    if a.cmd == "clocks":
        md = clocks_md(a.dir, a.kernels.split(","), a.title, a.command)
        if a.out:
            open(a.out, "w").write(md)
        print(md)
        return
    if a.cmd == "counters":
        md = counters_md(a.dirs, a.kernels.split(","), a.title, a.command)
        if a.out:
            open(a.out, "w").write(md)
        print(md)
        return
    if a.cmd == "stats":
        md = kernel_stats_md(a.csv, a.title, a.command)
        if a.out:
            open(a.out, "w").write(md)
        print(md)
    else:
        res = pmc_traffic(a.fetch, a.write, a.kernel, a.copy_bytes)
        res["command"] = a.command
        json.dump(res, open(a.out, "w"), indent=1)
        print(json.dumps(res, indent=1))


if __name__ == "__main__":
    main()
