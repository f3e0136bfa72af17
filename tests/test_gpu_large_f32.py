"""GPU parity past 32-bit element offsets in float32: Q, K, V, O and the
gradients hold 2^31 elements each (8 GiB), through the row-block forward
and the 16-row backward (64-blocks, d = 128). The same band layout and
local references as the 16-bit case: block row r of head h depends only on
key blocks r-1 and r, and the gradient of key block c only on query blocks
c and c+1. About 66 GiB of device memory.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, f64, max_abs

import block_sparse_matmul_amd as bsa

pytestmark = pytest.mark.gpu

Z, H, N, B, D = 1, 256, 65536, 64, 128
NB = N // B
SCALE = 1.0 / np.sqrt(D)


def _band():
    lay = np.zeros((NB, NB), np.uint8)
    r = np.arange(NB)
    lay[r, r] = 1
    lay[r[1:], r[1:] - 1] = 1
    return lay


@pytest.fixture(scope="module")
def big():
    props = torch.cuda.get_device_properties(0)
    if props.total_memory < 96 * 2**30:
        pytest.skip("needs about 66 GiB of device memory")
    announce("64-bit offsets: f32", Z, H, N, D)
    assert Z * H * N * D == 2**31
    g = torch.Generator(device="cuda").manual_seed(2025)
    q, k, v, do = (torch.randn((Z, H, N, D), generator=g, device="cuda") for _ in range(4))
    lay = _band()
    L = bsa.Layout(torch.from_numpy(np.ascontiguousarray(np.broadcast_to(lay, (H, NB, NB)))), B)
    nan = lambda: torch.full((Z, H, N, D), float("nan"), device="cuda")
    lse = torch.full((Z, H, N), float("nan"), device="cuda")
    o, lse = bsa.attention(L, q, k, v, SCALE, out=nan(), return_lse=True, lse=lse)
    dq, dk, dv = bsa.attention_backward_fused(L, q, k, v, o, lse, do, SCALE, out=(nan(), nan(), nan()))
    torch.cuda.synchronize()
    yield dict(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, lay=lay)
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


def _rows(t, h, b0, b1):
    return t[:, h:h + 1, b0 * B:b1 * B].cpu()


def test_every_output_written(big):
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert bool(torch.isfinite(big[name]).all()), name


CASES = [(h, r) for h in (0, 131, H - 1) for r in (0, NB // 2, NB - 1)]


@pytest.mark.parametrize("h,r", CASES)
def test_forward_and_backward_blocks(big, h, r):
    lo = max(r - 1, 0)
    sub = big["lay"][r:r + 1, lo:r + 1][None]
    q, do = _rows(big["q"], h, r, r + 1), _rows(big["do"], h, r, r + 1)
    k, v = _rows(big["k"], h, lo, r + 1), _rows(big["v"], h, lo, r + 1)
    assert max_abs(f64(_rows(big["o"], h, r, r + 1)), oracle.attention_dense(q, k, v, sub, B, SCALE)) <= TOL["f32"]
    lse = big["lse"][:, h:h + 1, r * B:(r + 1) * B].cpu()
    assert max_abs(f64(lse), oracle.attention_lse(q, k, sub, B, SCALE)) <= 1e-4
    rdq, _, _ = oracle.attention_backward_dense(q, k, v, do, sub, B, SCALE)
    assert max_abs(f64(_rows(big["dq"], h, r, r + 1)), rdq) <= TOL["f32"]
    # dK, dV of block column r: its rows r and r+1 with every key they see
    r1, khi = min(r + 2, NB), min(r + 2, NB)
    sub = big["lay"][r:r1, lo:khi][None]
    q, do = _rows(big["q"], h, r, r1), _rows(big["do"], h, r, r1)
    k, v = _rows(big["k"], h, lo, khi), _rows(big["v"], h, lo, khi)
    _, rdk, rdv = oracle.attention_backward_dense(q, k, v, do, sub, B, SCALE)
    c = (r - lo) * B
    for name, got, ref in (("dk", big["dk"], rdk), ("dv", big["dv"], rdv)):
        assert max_abs(f64(_rows(got, h, r, r + 1)), ref[:, :, c:c + B]) <= TOL["f32"], name
