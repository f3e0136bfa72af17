"""GPU parity of the 16-bit fused attention when a row's scores jump far
above the running max of its earlier key blocks, so that the exponentials
against that max reach 2^33 (accepted) or 2^64 and beyond, up to infinity
(the sub-step redone the exact way). Every query row is the same vector u
(|u|^2 = d); key block 0 holds small keys, key block 1 the keys f u, so the
scores of block 1 exceed block 0's by about f d scale log2(e) log2 units
(f = 2: 33; f = 5: 82; f = 40: 650). The expected values are the oracle's
float64 softmax; the bars are the 16-bit ones of the other parity tests.
The fp8 score operands (Q, K in OCP FP8 E4M3, V and O bf16) take the same
path after the score product; the oracle runs on the fp8 values.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, f64, max_abs, to_dev

import block_sparse_matmul_amd as bsa

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16}
F8 = torch.float8_e4m3fn


CASES = [(dt, b) for dt in ("bf16", "f16") for b in (64, 128)] + [("f8", 128)]


@pytest.mark.parametrize("dt,b", CASES)
@pytest.mark.parametrize("f", [2.0, 5.0, 40.0])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_far_above_the_running_max(dt, b, f, causal):
    d, H, nb, Z = 128, 2, 3, 1
    N = nb * b
    announce("score growth", dt, b, f, causal)
    g = torch.Generator("cpu").manual_seed(int(500 + b + 10 * f))
    u = torch.randn(d, generator=g)
    u = u / u.norm() * np.sqrt(d)
    q = u.expand(Z, H, N, d).clone()
    k = 0.01 * torch.randn((Z, H, N, d), generator=g)
    k[:, :, b:2 * b] = f * u  # block 1
    v = torch.randn((Z, H, N, d), generator=g)
    if dt == "f8":
        q, k, v = q.to(F8), k.to(F8), v.to(torch.bfloat16)
    else:
        q, k, v = (t.to(DT[dt]) for t in (q, k, v))
    lay = np.zeros((H, nb, nb), np.uint8)
    lay[:, :, 0] = 1          # every row sees block 0 first
    lay[:, 1:, 1] = 1         # rows 1, 2 then block 1 (on or below the diagonal)
    lay[:, 2, 2] = 1
    lay[1, 0, 0] = 1
    scale = 1.0 / np.sqrt(d)
    L = bsa.Layout(torch.from_numpy(lay), b)
    o, lse = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), scale, causal, return_lse=True)
    ref_o = oracle.attention_dense(q, k, v, lay, b, scale, causal)
    ref_l = oracle.attention_lse(q, k, lay, b, scale, causal)
    assert torch.isfinite(o).all()
    assert max_abs(f64(o), ref_o) <= TOL["bf16" if dt == "f8" else dt] * max(1.0, float(np.abs(ref_o).max()))
    bar = 1e-3 if dt == "f16" else 4e-3
    assert max_abs(f64(lse), ref_l) <= bar * max(1.0, float(np.abs(ref_l).max()))
