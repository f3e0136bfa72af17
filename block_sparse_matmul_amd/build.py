"""Build libbsattn.so (the HIP kernels and the C-ABI) in-tree for gfx950.

    python -m block_sparse_matmul_amd.build [--jobs N]

Each source under csrc/ is compiled to an object with hipcc in parallel, then
linked into block_sparse_matmul_amd/libbsattn.so. hipcc cross-compiles for
gfx950 without a GPU.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(HERE, "libbsattn.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "lut.hip", "sdd.hip", "softmax.hip", "dsd.hip", "dds.hip", "attention.hip",
           "attention_wide.hip", "attention_masked.hip", "attention_band.hip",
           "backward.hip", "backward_wide.hip"]

# Packed fp32 VALU forms are kept off (the compiler would otherwise fuse
# pairs of fp32 ops into v_pk_* instructions). MFMA results are kept in
# ordinary VGPRs: the softmax reads the score accumulators and rescales the
# output accumulators with VALU ops, which would otherwise copy them out of
# and back into AGPRs on every block.
COMMON = ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libbsattn.so)")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
