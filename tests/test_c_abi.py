"""The C ABI used from plain C99 programs (tests/c), with no Python in the
calling process: the header compiles as C and the library links and
validates arguments (CPU), and the fused attention runs from C on device
buffers of the HIP runtime, its O and row log-sum-exp checked against the
oracle (GPU)."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, announce, max_abs

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c", "bin")


def _binary(name):
    path = os.path.join(BIN, name)
    if not os.path.exists(path):  # built by the package build step; build here if missing
        sys.path.insert(0, os.path.join(HERE, "c"))
        import build_c
        build_c.build()
    return path


def test_c_program_validates_arguments_without_a_gpu():
    r = subprocess.run([_binary("abi_check")], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "abi_check ok" in r.stdout


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [False, True])
def test_c_program_runs_the_fused_attention(tmp_path, causal):
    Z, H, nb, b, d = 2, 2, 5, 64, 64
    N = nb * b
    lay = W.small_random_layout(H, nb, nb, 0.5, 950, force_diagonal=True)
    lay[1, 3, :] = 0  # an empty row
    g = torch.Generator("cpu").manual_seed(951)
    q, k, v = (torch.randn((Z, H, N, d), generator=g) for _ in range(3))
    scale = 0.125
    announce("C program attention", causal)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([Z, H, N, d, b, int(causal)], np.int32).tobytes())
        f.write(np.array([scale], np.float32).tobytes())
        f.write(np.ascontiguousarray(lay, np.uint8).tobytes())
        for t in (q, k, v):
            f.write(t.numpy().astype(np.float32).tobytes())
    r = subprocess.run([_binary("attn_run"), str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert f"nnz {int(lay.sum())}" in r.stdout
    out = np.fromfile(dst, np.float32)
    O = out[:Z * H * N * d].reshape(Z, H, N, d)
    lse = out[Z * H * N * d:].reshape(Z, H, N)
    assert max_abs(O, oracle.attention_dense(q, k, v, lay, b, scale, causal)) <= TOL["f32"]
    ref = oracle.attention_lse(q, k, lay, b, scale, causal)
    inf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(lse), inf)
    assert float(np.abs(lse[~inf].astype(np.float64) - ref[~inf]).max()) <= TOL["f32"]
