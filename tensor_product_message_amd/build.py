"""Build libconvtp.so (HIP, gfx950) in-tree with hipcc.

    python -m tensor_product_message_amd.build [--incremental]

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection switched off (-Xclang -target-feature -Xclang -packed-fp32-ops) and
no implicit multiply-add contraction (-ffp-contract=off: every fused
multiply-add is an explicit __builtin_fmaf in the source).
The convolution kernels are compiled once per degree triple (l_in, l_sh,
l_out), 64 objects from csrc/convtp_triple.hip with -DCTP_L1/-DCTP_L2/-DCTP_L3,
in parallel, largest first.  --incremental skips objects newer than every
source (for development; the default rebuilds everything).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libconvtp.so")
SOURCES = ["convtp_common.hip", "nodetp_kernels.hip", "graph_kernels.hip", "stream_probe.hip", "convtp_api.hip"]
TRIPLE_SOURCE = "convtp_triple.hip"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # fused multiply-adds only where the source writes __builtin_fmaf: the
         # compiler may not fuse a product into a later addition, so kernels
         # that share an arithmetic sequence (the backward's dY and the dY-only
         # kernel) round identically
         "-ffp-contract=off",
         "-Wall", "-Wno-unused-function", "-Wno-undefined-inline"]


def _paths(a: int, b: int, c: int) -> int:
    return sum(1 for p in range(a + 1) for q in range(b + 1) for r in range(c + 1) if abs(p - q) <= r <= p + q)


TRIPLES = sorted(((a, b, c) for a in range(4) for b in range(4) for c in range(4)),
                 key=lambda t: -_paths(*t))


def _compile(job) -> None:
    src, obj, defines = job
    cmd = [HIPCC, *FLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln
            and "is not a recognized feature for this target" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} {' '.join(defines)}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)


def _jobs(objdir: str):
    jobs = [(TRIPLE_SOURCE, os.path.join(objdir, f"triple_{a}{b}{c}.o"),
             [f"-DCTP_L1={a}", f"-DCTP_L2={b}", f"-DCTP_L3={c}"]) for a, b, c in TRIPLES]
    jobs += [(s, os.path.join(objdir, s.replace(".hip", ".o")), []) for s in SOURCES]
    return jobs


def build(verbose: bool = True, incremental: bool = False, workers: int = None) -> str:
    """Compile every HIP source and link libconvtp.so; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = _jobs(objdir)
    todo = jobs
    if incremental:
        headers = glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(HERE, "..", "include", "*.h"))
        newest_header = max(os.path.getmtime(p) for p in headers)

        def stale(job):
            src, obj, _ = job
            newest = max(newest_header, os.path.getmtime(os.path.join(CSRC, src)))
            return not os.path.exists(obj) or os.path.getmtime(obj) < newest
        todo = [j for j in jobs if stale(j)]
    n = workers or min(16, os.cpu_count() or 8)
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(_compile, todo))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *[j[1] for j in jobs]],
                   check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} ({len(todo)} of {len(jobs)} objects compiled)")
    return LIB


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv)
