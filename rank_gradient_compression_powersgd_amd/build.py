"""Build libpsgd.so in-tree with hipcc for gfx950.

    python -m rank_gradient_compression_powersgd_amd.build [--jobs N] [--verbose]

Every HIP source under csrc/ is compiled to an object file in csrc/_build/ and linked into
rank_gradient_compression_powersgd_amd/libpsgd.so. Packed fp32 instructions are disabled for
device code (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "libpsgd.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-I", INCLUDE,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(jobs: int = 0, verbose: bool = False, defines=(), out: str = "") -> str:
    """Compile every csrc/*.hip and link libpsgd.so (or `out`). `defines` are extra -D macros
    (kernel tile parameters) for alternative builds."""
    cc = hipcc()
    lib = os.path.abspath(out) if out else LIB
    bdir = BUILD if not defines else os.path.join(BUILD, "v_" + "_".join(d.replace("=", "") for d in defines))
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(bdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    dflags = [f"-D{d}" for d in defines]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [cc, *COMMON, *dflags, "-c", s, "-o", o], verbose) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--define", action="append", default=[], help="extra -D macro, e.g. K2_TC=2")
    ap.add_argument("--out", default="", help="output library path (default: in-tree libpsgd.so)")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose, a.define, a.out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
