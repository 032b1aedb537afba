"""Summaries of rocprofv3 output for the seam benchmark.

Turns the CSVs of three rocprofv3 runs of ``bench.py`` (``--kernel-trace
--stats``, ``--pmc FETCH_SIZE``, ``--pmc WRITE_SIZE``) into the short text
summaries kept under ``profiles/``.  HBM traffic per seam launch comes from
the two counters, each scaled by what the same counter reads for the
benchmark's own copy kernel, whose bytes are known exactly (it copies a
buffer of known size once per dispatch).

Usage: python -m layer_mhc_seam_amd.profiling TRACE_DIR FETCH_DIR WRITE_DIR
       OUT_STATS_MD OUT_TRAFFIC_MD [--head-stats-md MD --head-traffic-md MD]
       --cmd-trace "..." --cmd-fetch "..." --cmd-write "..."
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics

from .traffic import seam_bytes

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SRC = os.path.join(HERE, "csrc", "seam_kernels.hip")
HEAD_SRC = os.path.join(HERE, "csrc", "head_kernels.hip")
GEMM_SRC = os.path.join(HERE, "csrc", "gemm_kernels.hip")


def kernel_sha(src=KERNEL_SRC) -> str:
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def _one(pattern):
    files = glob.glob(pattern, recursive=True)
    if not files:
        raise FileNotFoundError(pattern)
    return files[0]


def kernel_stats(trace_dir):
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["Percentage"]))
            for r in rows]


def dispatch_us(trace_dir, name_part):
    """Durations (us) of each dispatch of the kernels whose name holds name_part."""
    rows = csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_trace.csv"))))
    return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows
            if name_part in r["Kernel_Name"]]


def is_headline(kernel_name):
    """The post-form, fp8-grid instantiation of the seam kernels (template
    arguments Form = 0, Out = 1); the benchmark also launches other forms."""
    return any(f"{k}<0, 1," in kernel_name for k in ("seam_rows_kernel", "seam_split_kernel"))


def is_head(kernel_name):
    return "head_reduce_kernel" in kernel_name


def is_gemm(kernel_name):
    return "mxfp8_gemm_kernel" in kernel_name


class Target:
    """One kernel to summarise: how to pick it out of the CSVs, its
    algorithmic read / write bytes per launch and the source it is built from."""

    def __init__(self, title, select, rd, wr, src):
        self.title, self.select, self.rd, self.wr, self.src = title, select, rd, wr, src


def seam_target(T=16384, H=5120, form="post", out_dtype="fp8_grid"):
    rd, wr = seam_bytes(T, H, form, out_dtype)
    return Target(f"seam, large prefill (T={T}, H={H}, post, fp8 grid)", is_headline, rd, wr,
                  KERNEL_SRC)


def head_target(T=16384, H=5120):
    return Target(f"head reduce (T={T}, H={H})", is_head, T * 4 * H * 2 + T * 16, T * H * 2,
                  HEAD_SRC)


def gemm_target(T=16384, N=5120, K=5120):
    """Algorithmic bytes: each operand and scale byte read once, out written."""
    return Target(f"MXFP8 GEMM (T={T}, N={N}, K={K})", is_gemm,
                  T * K + N * K + (T + N) * (K // 32), T * N * 2, GEMM_SRC)


def counter(dirname, name, select):
    """{"kernel" | "copy": [values per dispatch]} of one PMC counter."""
    out = {}
    for r in csv.DictReader(open(_one(os.path.join(dirname, "**", "*counter_collection.csv")))):
        if r["Counter_Name"] != name:
            continue
        k = r["Kernel_Name"]
        short = "kernel" if select(k) else "copy" if "copy_kernel" in k else None
        if short:
            out.setdefault(short, []).append(float(r["Counter_Value"]))
    return out


def summarize(trace_dir, fetch_dir, write_dir, tg, copy_target=None):
    """Kernel stats, per-dispatch durations and scaled traffic of target tg.
    The copy kernel's bytes per dispatch follow the seam's byte count (the
    benchmark sizes its copy from the headline seam)."""
    copy_target = copy_target or seam_target()
    stats = kernel_stats(trace_dir)
    fetch = counter(fetch_dir, "FETCH_SIZE", tg.select)
    write = counter(write_dir, "WRITE_SIZE", tg.select)
    copy_n = ((copy_target.rd + copy_target.wr) // 2 + 255) // 256 * 256
    f_copy = statistics.median(fetch["copy"]) * 1024
    w_copy = statistics.median(write["copy"]) * 1024
    f_scale, w_scale = copy_n / f_copy, copy_n / w_copy
    f_k = statistics.median(fetch["kernel"]) * 1024 * f_scale
    w_k = statistics.median(write["kernel"]) * 1024 * w_scale
    mine = [s for s in stats if tg.select(s[0])]
    top = max(mine, key=lambda r: r[1])[0]
    return dict(stats=stats, f_scale=f_scale, w_scale=w_scale, f_k=f_k, w_k=w_k,
                rd=tg.rd, wr=tg.wr, copy_n=copy_n, top=top, title=tg.title, src=tg.src,
                durations=dispatch_us(trace_dir, top))


def write_md(s, stats_md, traffic_md, cmds):
    with open(stats_md, "w") as f:
        f.write(f"# rocprofv3 kernel trace: {s['title']}\n\n")
        f.write("Command (repository root, MI355X):\n\n")
        f.write(f"    {cmds['trace']}\n\n")
        f.write("| kernel | calls | average us | % of GPU time |\n|---|---|---|---|\n")
        for name, calls, avg, pct in s["stats"][:9]:
            f.write(f"| `{name[:90]}` | {calls} | {avg / 1e3:.2f} | {pct:.1f} |\n")
        d = s["durations"]
        f.write(f"\nPer-dispatch durations of `{s['top'][:60]}` (us, launch order; the\n"
                f"first is the untimed output-allocating launch, then warmup and timed steps):\n\n")
        f.write("    " + " ".join(f"{x:.1f}" for x in d) + "\n\n")
        f.write(f"median {statistics.median(d):.1f} us, min {min(d):.1f} us\n")
    with open(traffic_md, "w") as f:
        f.write(f"# HBM traffic of one launch: {s['title']} (rocprofv3 FETCH_SIZE / WRITE_SIZE)\n\n")
        f.write("Commands (repository root, MI355X), one counter per run:\n\n")
        f.write(f"    {cmds['fetch']}\n    {cmds['write']}\n\n")
        f.write("Each counter is scaled by what it reads for the benchmark's copy kernel,\n")
        f.write(f"which moves {s['copy_n']} bytes each way per dispatch.\n\n")
        f.write(f"kernel_sha: {kernel_sha(s['src'])}\n")
        f.write(f"fetch_scale: {s['f_scale']:.4f}\n")
        f.write(f"write_scale: {s['w_scale']:.4f}\n")
        f.write(f"read_bytes_per_launch: {s['f_k']:.0f}\n")
        f.write(f"write_bytes_per_launch: {s['w_k']:.0f}\n")
        f.write(f"bytes_per_launch: {s['f_k'] + s['w_k']:.0f}\n")
        f.write(f"algorithmic_read_bytes: {s['rd']}\n")
        f.write(f"algorithmic_write_bytes: {s['wr']}\n")
        f.write(f"read_over_algorithmic: {s['f_k'] / s['rd']:.3f}\n")
        f.write(f"write_over_algorithmic: {s['w_k'] / s['wr']:.3f}\n")


def read_traffic(path):
    """key: value lines of a traffic summary (None if absent)."""
    if not os.path.exists(path):
        return None
    out = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", " ")):
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace_dir")
    ap.add_argument("fetch_dir")
    ap.add_argument("write_dir")
    ap.add_argument("stats_md")
    ap.add_argument("traffic_md")
    ap.add_argument("--head-stats-md")
    ap.add_argument("--head-traffic-md")
    ap.add_argument("--gemm-stats-md")
    ap.add_argument("--gemm-traffic-md")
    ap.add_argument("--cmd-trace", required=True)
    ap.add_argument("--cmd-fetch", required=True)
    ap.add_argument("--cmd-write", required=True)
    a = ap.parse_args()
    cmds = dict(trace=a.cmd_trace, fetch=a.cmd_fetch, write=a.cmd_write)
    write_md(summarize(a.trace_dir, a.fetch_dir, a.write_dir, seam_target()), a.stats_md,
             a.traffic_md, cmds)
    print(open(a.traffic_md).read())
    if a.head_stats_md:
        write_md(summarize(a.trace_dir, a.fetch_dir, a.write_dir, head_target()),
                 a.head_stats_md, a.head_traffic_md, cmds)
        print(open(a.head_traffic_md).read())
    if a.gemm_stats_md:
        write_md(summarize(a.trace_dir, a.fetch_dir, a.write_dir, gemm_target()),
                 a.gemm_stats_md, a.gemm_traffic_md, cmds)
        print(open(a.gemm_traffic_md).read())


if __name__ == "__main__":
    main()
