"""bs_attention_bwd_noalloc: the fused backward for callers that cannot
allocate, with D in the library's static device array, against
bs_attention_bwd (the caller-workspace entry point it shares its kernels
with) and against the oracle.

Two calls in a row, the second on a smaller problem, so that the second call
runs on the array the first one left behind; then a size past the array's
limit, which the library rejects on the host before any launch.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, announce, f64, max_abs, to_dev

import block_sparse_matmul_amd as bsa
from block_sparse_matmul_amd import _lib

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
SCRATCH_ROWS = 1 << 21


def _grad_tol(dt, ref):
    return TOL["f32"] if dt == "f32" else TOL[dt] * max(1.0, float(np.abs(ref).max()))


def _case(Z, H, nb, b, d, dt, causal, seed):
    lay = W.small_random_layout(H, nb, nb, 0.5, seed, force_diagonal=True)
    g = torch.Generator("cpu").manual_seed(seed + 1)
    q, k, v, do = [torch.randn((Z, H, nb * b, d), generator=g).to(DT[dt]) for _ in range(4)]
    return lay, q, k, v, do


@pytest.mark.parametrize("dt,b,d,causal", [("f32", 64, 64, True), ("bf16", 128, 128, False)])
def test_noalloc_matches_workspace_entry_point_two_calls(dt, b, d, causal):
    # first call larger, second smaller: the second reuses (and must not
    # depend on) what the first left in the static array
    for n, (Z, H, nb) in enumerate(((2, 3, 6), (1, 2, 3))):
        announce("noalloc bwd", dt, b, d, causal, "call", n, (Z, H, nb))
        lay, q, k, v, do = _case(Z, H, nb, b, d, dt, causal, 900 + 10 * n + b)
        L = bsa.Layout(torch.from_numpy(lay), b)
        qd, kd, vd, dod = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
        o, lse = bsa.attention(L, qd, kd, vd, 0.125, causal, return_lse=True)
        ref = bsa.attention_backward_fused(L, qd, kd, vd, o, lse, dod, 0.125, causal)
        outs = tuple(torch.full_like(t, float("nan")) for t in (qd, kd, vd))
        got = bsa.attention_backward_fused(L, qd, kd, vd, o, lse, dod, 0.125, causal, out=outs, noalloc=True)
        torch.cuda.synchronize()
        for name, a, r in zip(("dq", "dk", "dv"), got, ref):
            assert not torch.isnan(a).any(), name
            assert max_abs(f64(a), f64(r)) <= TOL[dt], name
            assert torch.equal(a, r), name  # same kernels, same D: bit-identical
        dense = oracle.attention_backward_dense(q, k, v, do, lay, b, 0.125, causal)
        for name, a, r in zip(("dq", "dk", "dv"), got, dense):
            assert max_abs(f64(a), r) <= _grad_tol(dt, r), name


def test_noalloc_rejects_rows_beyond_the_static_buffer():
    # Z*H*nbr*b = (2^17 + 1) * 16 > 2^21: refused on the host, nothing runs
    Z, b, d = (SCRATCH_ROWS // 16) + 1, 16, 64
    announce("noalloc bwd limit", Z)
    L = bsa.Layout(torch.ones((1, 1, 1), dtype=torch.uint8), b)
    shape = (Z, 1, b, d)
    q, k, v, o, do = [torch.empty(shape, device="cuda") for _ in range(5)]
    lse = torch.empty((Z, 1, b), device="cuda")
    with pytest.raises(bsa.BsError) as e:
        bsa.attention_backward_fused(L, q, k, v, o, lse, do, 0.125, noalloc=True)
    assert e.value.code == _lib.BS_ERR_SHAPE
    assert b"static D buffer" in _lib.lib().bs_last_error()
