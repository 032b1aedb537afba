"""Summaries of rocprofv3 output of ``bench.py`` runs.

Turns the CSVs of three rocprofv3 runs (``--kernel-trace --stats``, ``--pmc
FETCH_SIZE``, ``--pmc WRITE_SIZE``) into the short text summaries kept under
``profiles/``.  HBM traffic per launch comes from the two counters, each
scaled by what the same counter reads for the benchmark's calibration copy
(the first three copy-kernel dispatches of every run, 256 MiB each way),
whose bytes are known exactly.

Usage:
  python -m layer_mhc_seam_amd.profiling seam WORKLOAD TRACE_DIR FETCH_DIR WRITE_DIR
      --cmd-trace "..." --cmd-fetch "..." --cmd-write "..."
  python -m layer_mhc_seam_amd.profiling head|gemm TRACE_DIR FETCH_DIR WRITE_DIR --cmd-...
writes profiles/kernel_trace_<kernel>_<workload>.md and profiles/traffic_<...>.md.
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


def seam_select(form, out):
    """Seam kernel instances of one form and out_dtype (template arguments
    Form, Out): whole-row (with its split tail) and split launches."""
    def sel(kernel_name):
        return any(f"{k}<{form}, {out}," in kernel_name
                   for k in ("seam_rows_kernel", "seam_split_kernel"))
    return sel


def is_head(kernel_name):
    return "head_reduce_kernel" in kernel_name


def is_gemm(kernel_name):
    """The 256 x 256 block instance, which T = 16384, N = K = 5120 takes (the
    benchmark also runs the smaller block shapes at few tokens)."""
    return "mxfp8_gemm_tile_kernel" in kernel_name and "Tile<256, 256," in kernel_name


class Target:
    """One kernel to summarise: how to pick it out of the CSVs, its
    algorithmic read / write bytes per launch and the source it is built from."""

    def __init__(self, title, select, rd, wr, src):
        self.title, self.select, self.rd, self.wr, self.src = title, select, rd, wr, src


def seam_target(name):
    from . import synth
    from .seam import FORMS, OUT_DTYPES
    w = synth.WORKLOADS[name]
    rd, wr = seam_bytes(w.T, w.H, w.form, w.out_dtype)
    return Target(f"seam {name} (T={w.T}, H={w.H}, {w.form}, {w.out_dtype})",
                  seam_select(FORMS[w.form], OUT_DTYPES[w.out_dtype]), rd, wr, KERNEL_SRC)


def head_target(T=16384, H=5120):
    return Target(f"head reduce (T={T}, H={H})", is_head, T * 4 * H * 2 + T * 16, T * H * 2,
                  HEAD_SRC)


def gemm_target(T=16384, N=5120, K=5120):
    """Algorithmic bytes: each operand and scale byte read once, out written."""
    return Target(f"MXFP8 GEMM (T={T}, N={N}, K={K})", is_gemm,
                  T * K + N * K + (T + N) * (K // 32), T * N * 2, GEMM_SRC)


CALIB_BYTES = 256 << 20    # bench.py's calibration copy, bytes each way per dispatch


def counter(dirname, name, select):
    """{"kernel": [values per dispatch of the selected kernel], "copy": [values
    of the first three copy-kernel dispatches]} of one PMC counter."""
    rows = [r for r in csv.DictReader(open(_one(os.path.join(dirname, "**",
                                                                "*counter_collection.csv"))))
            if r["Counter_Name"] == name]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    out = {"kernel": [], "copy": []}
    for r in rows:
        k = r["Kernel_Name"]
        if select(k):
            out["kernel"].append(float(r["Counter_Value"]))
        elif "copy_kernel" in k and len(out["copy"]) < 3:
            out["copy"].append(float(r["Counter_Value"]))
    return out


def summarize(trace_dir, fetch_dir, write_dir, tg):
    """Kernel stats, per-dispatch durations and scaled traffic of target tg."""
    stats = kernel_stats(trace_dir)
    fetch = counter(fetch_dir, "FETCH_SIZE", tg.select)
    write = counter(write_dir, "WRITE_SIZE", tg.select)
    copy_n = CALIB_BYTES
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


def short_name(name, width=90):
    """A kernel name without namespaces, 'void' and its argument list."""
    n = name.replace("mhc::(anonymous namespace)::", "").replace("mhc::", "")
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):   # cut at the argument list (the first '(' outside <>)
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            n = n[:i]
            break
    return n[:width]


def write_md(s, stats_md, traffic_md, cmds):
    with open(stats_md, "w") as f:
        f.write(f"# rocprofv3 kernel trace: {s['title']}\n\n")
        f.write("Command (repository root, MI355X):\n\n")
        f.write(f"    {cmds['trace']}\n\n")
        f.write("| kernel | calls | average us | % of GPU time |\n|---|---|---|---|\n")
        for name, calls, avg, pct in s["stats"][:12]:
            f.write(f"| `{short_name(name)}` | {calls} | {avg / 1e3:.2f} | {pct:.1f} |\n")
        d = s["durations"]
        if s["title"].startswith("seam"):
            order = ("launch order: the\npriming seam where it is the same kernel (post form, "
                     "bf16), the untimed\noutput-allocating launch, then warmup and timed steps")
        else:
            order = "launch order: the\nuntimed first launches, then warmup and timed ones"
        f.write(f"\nPer-dispatch durations of `{short_name(s['top'])}` (us, {order}):\n\n")
        f.write("    " + " ".join(f"{x:.1f}" for x in d) + "\n\n")
        f.write(f"median {statistics.median(d):.1f} us, min {min(d):.1f} us\n")
    with open(traffic_md, "w") as f:
        f.write(f"# HBM traffic of one launch: {s['title']} (rocprofv3 FETCH_SIZE / WRITE_SIZE)\n\n")
        f.write("Commands (repository root, MI355X), one counter per run:\n\n")
        f.write(f"    {cmds['fetch']}\n    {cmds['write']}\n\n")
        f.write("Each counter is scaled by what it reads for the benchmark's calibration copy\n")
        f.write(f"(the run's first three copy-kernel dispatches, {s['copy_n']} bytes each way).\n\n")
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
    ap.add_argument("kind", choices=("seam", "head", "gemm"))
    ap.add_argument("rest", nargs="+", help="[WORKLOAD] TRACE_DIR FETCH_DIR WRITE_DIR")
    ap.add_argument("--cmd-trace", required=True)
    ap.add_argument("--cmd-fetch", required=True)
    ap.add_argument("--cmd-write", required=True)
    ap.add_argument("--out-dir", default=os.path.join(os.path.dirname(HERE), "profiles"))
    a = ap.parse_args()
    cmds = dict(trace=a.cmd_trace, fetch=a.cmd_fetch, write=a.cmd_write)
    if a.kind == "seam":
        name, trace_dir, fetch_dir, write_dir = a.rest
        tg, tag = seam_target(name), f"seam_{name}"
    elif a.kind == "head":
        trace_dir, fetch_dir, write_dir = a.rest
        tg, tag = head_target(), "head_reduce_prefill16k"
    else:
        trace_dir, fetch_dir, write_dir = a.rest
        tg, tag = gemm_target(), "mxfp8_gemm_16384x5120x5120"
    stats_md = os.path.join(a.out_dir, f"kernel_trace_{tag}.md")
    traffic_md = os.path.join(a.out_dir, f"traffic_{tag}.md")
    write_md(summarize(trace_dir, fetch_dir, write_dir, tg), stats_md, traffic_md, cmds)
    print(open(traffic_md).read())


if __name__ == "__main__":
    main()
