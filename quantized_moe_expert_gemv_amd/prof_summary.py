"""Condense rocprofv3 CSV output into the short text summaries kept with the
library's measurements.

    python -m quantized_moe_expert_gemv_amd.prof_summary stats OUT.md CMD KERNEL_STATS_CSV
    python -m quantized_moe_expert_gemv_amd.prof_summary traffic OUT.md CMD_FETCH CMD_WRITE \
        FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV COPY_BYTES
    python -m quantized_moe_expert_gemv_amd.prof_summary mfma OUT.md CMD PMC_CSV N_CU

`stats` lists every kernel of a `--kernel-trace --stats` run (calls, average
and total time).  `traffic` takes two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE`
runs of a workload and of a plain device copy of COPY_BYTES bytes each way;
the copy gives the bytes each counter unit stands for, so a kernel's HBM
bytes per dispatch = mean counter value x that factor.  The summary ends with
one `traffic:` line per library kernel (and the hash of the kernel sources the
counters were taken on), which the benchmark reads.  `mfma` takes one `--pmc`
run of the matrix-core counters (SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA,
SQ_INSTS_VALU, SQ_INSTS_VALU_MFMA_MOPS_F16/BF16, SQ_BUSY_CYCLES,
GRBM_GUI_ACTIVE) and writes, per kernel, the fraction of SIMD cycles the
matrix cores were busy, the MFMA flops the hardware counted and the VALU
instructions issued per MFMA, ending with one `mfma:` line per kernel.
"""

import csv
import hashlib
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

# library kernel name fragment -> benchmark name
KERNELS = [("k_route_gemv", "route_gemv"), ("k_topk", "topk"), ("k_topk_block", "topk"),
           ("k_topk_block_decode", "topk"), ("k_gateup", "gateup"), ("k_down", "down_combine"),
           ("k_down16", "down_combine"), ("k_router", "router_gemm"), ("k_topk_chunks", "topk"),
           ("k_colscan", "colscan"), ("k_scan", "scan"), ("k_scatter", "scatter"), ("k_gemm_gateup", "gateup_gemm"),
           ("k_gemm_down", "down_gemm"), ("k_combine", "combine")]


# the sources each path's kernels are built from (a counter summary stays
# valid while these are unchanged)
PATH_SOURCES = {"decode": ("common.hpp", "decode.hip", "kernels.hpp"),
                "prefill": ("common.hpp", "kernels.hpp", "prefill.hip")}
DECODE_KERNELS = ("k_route_gemv", "k_topk", "k_topk_block", "k_topk_block_decode", "k_permute", "k_gateup", "k_down",
                  "k_down16")


def source_hash(path=None):
    """sha256 over the kernel sources of one path (all csrc/*.hip, *.hpp when
    path is None), in name order."""
    h = hashlib.sha256()
    d = os.path.join(HERE, "csrc")
    names = PATH_SOURCES[path] if path else [n for n in os.listdir(d) if n.endswith((".hip", ".hpp"))]
    for name in sorted(names):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def kernel_path(kernel):
    m = re.search(r"::(k_[A-Za-z0-9_]+)", kernel)
    return "decode" if m and m.group(1) in DECODE_KERNELS else "prefill"


def bench_name(kernel):
    m = re.search(r"::(k_[A-Za-z0-9_]+)", kernel)
    if not m:
        return None
    return dict(KERNELS).get(m.group(1))


def read_stats(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def stats(out, cmd, stats_csv):
    rows = read_stats(stats_csv)
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "    " + cmd, "",
             "| kernel | calls | avg us | total ms | % |", "|---|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"]
        short = name if len(name) < 90 else name[:87] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    lines += ["", f"kernel sources: decode {source_hash('decode')}, prefill {source_hash('prefill')}", ""]
    open(out, "w").write("\n".join(lines))


def per_kernel_counter(path):
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def traffic(out, cmd_f, cmd_w, fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_bytes):
    copy_bytes = int(copy_bytes)
    f = per_kernel_counter(fetch_csv)
    w = per_kernel_counter(write_csv)

    def copy_factor(path):
        vals = [v for k, vs in per_kernel_counter(path).items() if "copyBuffer" in k or "copy" in k.lower()
                for v in vs]
        vals = sorted(vals)[-4:]                  # the timed copies (largest dispatches)
        return copy_bytes / (sum(vals) / len(vals))

    ff, fw = copy_factor(cfetch_csv), copy_factor(cwrite_csv)
    lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands:", "", "    " + cmd_f, "    " + cmd_w, "",
             f"Calibration: a plain device copy of {copy_bytes} bytes each way reads "
             f"{copy_bytes / ff:.0f} KiB of FETCH_SIZE and {copy_bytes / fw:.0f} KiB of "
             f"WRITE_SIZE: bytes per counter KiB = {ff:.4f} (fetch), {fw:.4f} (write).", "",
             "| kernel | dispatches | FETCH KiB | WRITE KiB | HBM bytes / dispatch |", "|---|---:|---:|---:|---:|"]
    tagged = []
    for k in sorted(f):
        name = bench_name(k)
        fv = f[k]
        wv = w.get(k, [0.0])
        fm, wm = sum(fv) / len(fv), sum(wv) / len(wv)
        b = fm * ff + wm * fw
        short = k if len(k) < 70 else k[:67] + "..."
        lines.append(f"| `{short}` | {len(fv)} | {fm:.1f} | {wm:.1f} | {b:.0f} |")
        if name:
            tagged.append((name, kernel_path(k), b, len(fv)))
    lines += ["", f"kernel sources: decode {source_hash('decode')}, prefill {source_hash('prefill')}", ""]
    merged = {}
    for name, kp, b, n in tagged:           # several instantiations of one kernel: dispatch-weighted mean
        tb, tn = merged.get((name, kp), (0.0, 0))
        merged[(name, kp)] = (tb + b * n, tn + n)
    for (name, kp), (tb, tn) in sorted(merged.items()):
        lines.append(f"traffic: kernel={name} path={kp} bytes_per_dispatch={tb / tn:.0f} "
                     f"sources={source_hash(kp)}")
    lines.append("")
    open(out, "w").write("\n".join(lines))


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_VALU_MFMA_MOPS_F16",
                 "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
N_XCC = 8                  # GRBM_GUI_ACTIVE is summed over the accelerator dies


def per_kernel_counters(path):
    """{kernel: {counter: [value per dispatch]}} of a multi-counter pmc CSV."""
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return acc


def mfma(out, cmd, pmc_csv, n_cu):
    """Matrix-core utilisation per kernel: busy = SQ_VALU_MFMA_BUSY_CYCLES
    (summed over SIMDs) / (GRBM_GUI_ACTIVE / N_XCC cycles x 4 SIMDs x n_cu);
    flops = (MOPS_F16 + MOPS_BF16) x 512; VALU per MFMA = SQ_INSTS_VALU /
    SQ_INSTS_MFMA (the MFMAs are counted among the VALU instructions, so the
    plain VALU work is SQ_INSTS_VALU - SQ_INSTS_MFMA)."""
    n_cu = int(n_cu)
    acc = per_kernel_counters(pmc_csv)
    lines = ["# Matrix-core counters per dispatch (rocprofv3 --pmc)", "", "Command:", "", "    " + cmd, "",
             f"Busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {N_XCC} x 4 SIMDs x {n_cu} CUs); "
             "flops = (SQ_INSTS_VALU_MFMA_MOPS_F16 + _BF16) x 512; VALU/MFMA = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / "
             "SQ_INSTS_MFMA.", "",
             "| kernel | dispatches | GUI cycles / die | MFMA busy cycles | MFMA busy | MFMA insts | MFMA GFLOP "
             "| other VALU / MFMA |", "|---|---:|---:|---:|---:|---:|---:|---:|"]
    tagged = {}
    for k in sorted(acc):
        c = {n: (sum(v) / len(v) if v else 0.0) for n, v in acc[k].items()}
        if not c.get("SQ_INSTS_MFMA"):
            continue
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCC
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        frac = busy / (gui * 4 * n_cu) if gui else 0.0
        flops = (c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)) * 512
        other = (c.get("SQ_INSTS_VALU", 0.0) - c["SQ_INSTS_MFMA"]) / c["SQ_INSTS_MFMA"]
        short = k if len(k) < 70 else k[:67] + "..."
        n = len(next(iter(acc[k].values())))
        lines.append(f"| `{short}` | {n} | {gui:.0f} | {busy:.4g} | {frac:.3f} | {c['SQ_INSTS_MFMA']:.4g} | "
                     f"{flops / 1e9:.2f} | {other:.2f} |")
        name = bench_name(k)
        if name:
            tb = tagged.setdefault((name, kernel_path(k)), [0.0, 0.0, 0.0, 0])
            tb[0] += frac * n; tb[1] += flops * n; tb[2] += other * n; tb[3] += n
    lines += ["", f"kernel sources: decode {source_hash('decode')}, prefill {source_hash('prefill')}", ""]
    for (name, kp), (fr, fl, ot, n) in sorted(tagged.items()):
        lines.append(f"mfma: kernel={name} path={kp} busy_frac={fr / n:.4f} mfma_flops={fl / n:.0f} "
                     f"valu_per_mfma={ot / n:.3f} sources={source_hash(kp)}")
    lines.append("")
    open(out, "w").write("\n".join(lines))


def read_mfma(path):
    """{bench kernel name: {busy_frac, mfma_flops, valu_per_mfma}} from a
    matrix-core counter summary, or {} when missing or taken on other kernel
    sources."""
    if not os.path.exists(path):
        return {}
    cur = {p: source_hash(p) for p in PATH_SOURCES}
    res = {}
    for line in open(path):
        if line.startswith("mfma:"):
            kv = dict(p.split("=", 1) for p in line.split()[1:])
            if kv.get("path") in cur and kv.get("sources") == cur[kv["path"]]:
                res[kv["kernel"]] = {"busy_frac": float(kv["busy_frac"]), "mfma_flops": float(kv["mfma_flops"]),
                                     "valu_per_mfma": float(kv["valu_per_mfma"])}
    return res


def read_traffic(path):
    """{bench kernel name: bytes per dispatch} from a traffic summary, or {}
    when it is missing or was taken on other kernel sources."""
    if not os.path.exists(path):
        return {}
    cur = {p: source_hash(p) for p in PATH_SOURCES}
    res = {}
    for line in open(path):
        if line.startswith("traffic:"):
            kv = dict(p.split("=", 1) for p in line.split()[1:])
            if kv.get("path") in cur and kv.get("sources") == cur[kv["path"]]:
                res[kv["kernel"]] = float(kv["bytes_per_dispatch"])
    return res


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "stats":
        stats(*sys.argv[2:5])
    elif mode == "traffic":
        traffic(*sys.argv[2:11])
    elif mode == "mfma":
        mfma(*sys.argv[2:6])
    elif mode == "hash":
        print(source_hash(sys.argv[2] if len(sys.argv) > 2 else None))
    else:
        sys.exit(f"unknown mode {mode}")
