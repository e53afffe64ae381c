"""Build libmoegg.so (HIP, gfx950) in-tree.

    python -m token_routing_amd.build [--report]

Each .hip source under csrc/ is compiled with hipcc for gfx950 only, with
packed-fp32 instruction selection disabled, and linked into
token_routing_amd/libmoegg.so.  --report prints the compiler's per-kernel
resource usage (VGPRs, AGPRs, spills, LDS, occupancy).
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoegg.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]

SOURCES = ["route.hip", "gemm.hip", "generic.hip", "combine.hip", "api.hip"]


def _compile(src: str, report: bool, defines=(), build_dir=BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    if report:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    if report:
        sys.stdout.write(res.stderr)
    return obj


def build(report: bool = False, defines=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile and link; `defines` are extra -D settings (tile-shape macros)."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, report, defines, build_dir), SOURCES))
    tmp = out + ".tmp"
    subprocess.check_call([HIPCC, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--report", action="store_true")
    print(build(report=ap.parse_args().report))
