"""Compile the plain-C programs of tests/c against include/bsattn.h and the
in-tree libbsattn.so (gcc, C99): abi_check (argument validation, no GPU)
and attn_run (the fused attention through the C ABI on the GPU). The
binaries go to tests/c/bin and find the library through a relative rpath."""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "bin")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> None:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C ABI test programs")
    os.makedirs(BIN, exist_ok=True)
    common = ["-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
              "-L", os.path.join(ROOT, "block_sparse_matmul_amd"), "-Wl,-rpath,$ORIGIN/../../../block_sparse_matmul_amd"]
    progs = {
        "abi_check": ([], ["-lbsattn"]),
        "attn_run": (["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")],
                     ["-lbsattn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"]),
    }
    for name, (pre, libs) in progs.items():
        cmd = [cc] + common + pre + [os.path.join(HERE, name + ".c"), "-o", os.path.join(BIN, name)] + libs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)


if __name__ == "__main__":
    build(verbose=True)
