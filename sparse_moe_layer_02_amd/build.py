"""Compile the HIP library in-tree for gfx950: ``libmoe_mi355x.so``.

Each ``csrc/*.hip`` is compiled to an object in parallel, then linked.  Packed
fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmoe_mi355x.so")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, out: str = OUT, defines=()) -> str:
    """Compile every csrc/*.hip and link them into ``out``.  ``defines`` are
    extra -D options (tuning variants; the default build uses none)."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="moe_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *FLAGS, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            if verbose:
                print("compiled", os.path.basename(src), flush=True)
            return obj

        with ThreadPoolExecutor(max(1, min(len(srcs), os.cpu_count() or 1, 16))) as ex:
            objs = list(ex.map(compile_one, srcs))
        tmp_out = out + f".tmp{os.getpid()}"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_out, out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    out = OUT
    if "-o" in args:
        out = os.path.abspath(args[args.index("-o") + 1])
    defs = [a[2:] for a in args if a.startswith("-D")]
    print(build(verbose="-v" in args, out=out, defines=defs))
