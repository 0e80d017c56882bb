"""Build libattnq.so (HIP, gfx950) in-tree: paged_kv_amd/libattnq.so.

Usage:  python -m paged_kv_amd.build  [--jobs N]

Every .hip source in csrc/ is compiled for gfx950 only, then linked into one
shared library.  Packed-fp32 instruction selection is disabled for all device
code; the RoPE file additionally forbids fused multiply-add contraction, its
arithmetic being defined product by product.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattnq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
PER_FILE = {
    "rope.hip": ["-ffp-contract=off"],
    "quant.hip": ["-ffp-contract=off"],
}


def sources():
    return sorted(f for f in os.listdir(SRC) if f.endswith(".hip"))


def _compile(name: str) -> str:
    src = os.path.join(SRC, name)
    obj = os.path.join(OUT_DIR, name[:-4] + ".o")
    cmd = [HIPCC, *COMMON, *PER_FILE.get(name, []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    names = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, names))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {', '.join(names)}")
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args(argv)
    build(a.jobs, verbose=True)


if __name__ == "__main__":
    sys.exit(main())
