"""Runtime behaviour on the GPU: stream ordering and the allocation-failure
path.

* Stream ordering: every compute call is asynchronous on the caller's
  stream. A side stream first waits (a spin kernel), then overwrites the
  query tensor, then runs the fused attention; the result must be that of
  the new queries, which holds only if the attention ran after the copy on
  that same stream.
* Allocation failure: with BS_FAULT_INJECT=oom the layout build fails with
  BS_ERR_OOM before any allocation is attempted, returns no handle, and the
  next build without the variable succeeds. No GPU fault is involved.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, announce, f64, max_abs, to_dev

import block_sparse_matmul_amd as bsa
from block_sparse_matmul_amd import _lib

pytestmark = pytest.mark.gpu


def test_calls_follow_the_callers_stream():
    announce("stream ordering")
    H, nb, b, d, Z = 2, 8, 64, 64, 2
    lay = W.small_random_layout(H, nb, nb, 0.4, 31, force_diagonal=True)
    g = torch.Generator("cpu").manual_seed(32)
    q_old, q_new, k, v = [torch.randn((Z, H, nb * b, d), generator=g) for _ in range(4)]
    L = bsa.Layout(torch.from_numpy(lay), b)
    qd, qn, kd, vd = to_dev(q_old), to_dev(q_new), to_dev(k), to_dev(v)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(20_000_000)  # keep the side stream busy before the copy
        qd.copy_(qn)
        o = bsa.attention(L, qd, kd, vd, 0.125)
        s = bsa.sdd(L, qd, kd)
    side.synchronize()
    ref = oracle.attention_dense(q_new, k, v, lay, b, 0.125)
    assert max_abs(f64(o), ref) <= TOL["f32"]
    lut = oracle.lut_from_layout(lay)
    assert max_abs(f64(s), oracle.sdd(q_new, k, lay, b)) <= TOL["f32"]
    assert s.shape[1] == int(lut["row_ptr"][-1])


def test_oom_injection_fails_cleanly_and_recovers():
    announce("oom injection")
    lay = np.ones((1, 2, 2), np.uint8)
    os.environ["BS_FAULT_INJECT"] = "oom"
    try:
        with pytest.raises(bsa.BsError) as e:
            bsa.Layout(torch.from_numpy(lay), 16)
        assert e.value.code == _lib.BS_ERR_OOM
        with pytest.raises(bsa.BsError) as e2:
            bsa.Layout.acsr([(0, 2, 1, 0, 1, 1)], 1, 2, 2, 16)
        assert e2.value.code == _lib.BS_ERR_OOM
    finally:
        del os.environ["BS_FAULT_INJECT"]
    L = bsa.Layout(torch.from_numpy(lay), 16)
    assert L.nnz == 4
