"""GPU parity of the three modes with transposed operands (bs_sdd_ex,
bs_dsd_ex, bs_dds_ex) against the oracle, which is given the operands the
way the method uses them (the stored arrays with their last two axes
swapped where a flag says so). Tolerances as for the plain calls: fp32
1e-4; bf16 outputs 2e-2 (SDD outputs are fp32 from exact bf16 products:
1e-4)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, announce, f64, max_abs, to_dev

import block_sparse_matmul_amd as bsa

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
FLAGS = [(True, False), (False, True), (True, True)]


def _dense(shape, seed, dt):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g).to(DT[dt])


def _blocks(Z, nnz, b, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.rand((Z, nnz, b, b), generator=g) / b


def _t(x):
    return x.transpose(-1, -2).contiguous()


@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("K", [64, 48])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("ta,tb", FLAGS)
def test_sdd_transposed(b, K, dt, ta, tb):
    H, nbr, nbc, Z = 2, 3, 4, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 500 + b + K)
    lay[0, 1, :] = 0
    announce("sdd transposed", b, K, dt, ta, tb)
    a = _dense((Z, H, nbr * b, K), 501, dt)
    bb = _dense((Z, H, nbc * b, K), 502, dt)
    L = bsa.Layout(torch.from_numpy(lay), b)
    S = bsa.sdd(L, to_dev(_t(a) if ta else a), to_dev(_t(bb) if tb else bb), trans_a=ta, trans_b=tb)
    assert max_abs(f64(S), oracle.sdd(a, bb, lay, b)) <= TOL["f32"]


@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("Nd", [64, 48])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("ta,tb", FLAGS)
def test_dsd_transposed(b, Nd, dt, ta, tb):
    H, nbr, nbc, Z = 2, 3, 4, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 510 + b + Nd)
    lay[1, 2, :] = 0
    lay[0, :, 1] = 0
    nnz = int(lay.sum())
    announce("dsd transposed", b, Nd, dt, ta, tb)
    n_in = (nbr if ta else nbc) * b
    B = _dense((Z, H, n_in, Nd), 511, dt)
    P = _blocks(Z, nnz, b, 512)
    L = bsa.Layout(torch.from_numpy(lay), b)
    C = bsa.dsd(L, to_dev(P), to_dev(_t(B) if tb else B), trans_a=ta, trans_b=tb)
    ref = oracle.dsd_t(P, B, lay, b) if ta else oracle.dsd(P, B, lay, b)
    assert C.dtype == B.dtype
    assert max_abs(f64(C), ref) <= TOL[dt]


@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("M", [32, 48])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("ta,tb", FLAGS)
def test_dds_transposed(b, M, dt, ta, tb):
    H, nbr, nbc, Z = 2, 3, 5, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 520 + b + M)
    lay[0, :, 2] = 0
    lay[1, 1, :] = 0
    nnz = int(lay.sum())
    announce("dds transposed", b, M, dt, ta, tb)
    n_in = (nbc if tb else nbr) * b
    A = _dense((Z, H, M, n_in), 521, dt)
    S = _blocks(Z, nnz, b, 522)
    L = bsa.Layout(torch.from_numpy(lay), b)
    C = bsa.dds(L, to_dev(_t(A) if ta else A), to_dev(S), trans_a=ta, trans_b=tb)
    ref = oracle.dds_t(A, S, lay, b) if tb else oracle.dds(A, S, lay, b)
    assert max_abs(f64(C), ref) <= TOL[dt]


def test_dsd_transposed_blocks_fast_path_is_dsd_t():
    """trans_a with Nd of 64 or 128 runs the DSD^T kernel of the backward:
    the same bits as dsd_t."""
    b, H, nb, Z, Nd = 32, 2, 4, 2, 64
    lay = W.small_random_layout(H, nb, nb, 0.5, 530)
    announce("dsd trans_a fast path")
    B = to_dev(_dense((Z, H, nb * b, Nd), 531, "f32"))
    P = to_dev(_blocks(Z, int(lay.sum()), b, 532))
    L = bsa.Layout(torch.from_numpy(lay), b)
    assert torch.equal(bsa.dsd(L, P, B, trans_a=True), bsa.dsd_t(L, P, B))


def test_transpose_flag_errors():
    import ctypes as C
    from block_sparse_matmul_amd import _lib
    lay = np.ones((1, 2, 2), np.uint8)
    announce("transpose flag errors")
    L = bsa.Layout(torch.from_numpy(lay), 16)
    a = torch.zeros((1, 1, 32, 64), device="cuda")
    s = torch.zeros((1, 4, 16, 16), device="cuda")
    p = lambda t: C.c_void_p(t.data_ptr())
    assert _lib.lib().bs_sdd_ex(L.handle, p(a), p(a), p(s), 1, 64, 4, _lib.BS_F32, None) == _lib.BS_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        bsa.sdd(L, a, a, trans_a=True)  # a would have to be [1, 1, K, 32]


def test_transposed_modes_on_an_empty_layout():
    """No stored block: SDD writes nothing, DSD and DDS write zeros."""
    b, H, nb, Z = 16, 2, 3, 2
    lay = np.zeros((H, nb, nb), np.uint8)
    announce("transposed modes empty layout")
    L = bsa.Layout(torch.from_numpy(lay), b)
    B = to_dev(_dense((Z, H, 48, nb * b), 540, "f32"))
    P = torch.zeros((Z, 0, b, b), device="cuda")
    for ta in (False, True):
        C = bsa.dsd(L, P, B, trans_a=ta, trans_b=True)
        assert C.shape == (Z, H, nb * b, 48) and torch.all(C == 0)
        D = bsa.dds(L, B, P, trans_a=False, trans_b=True) if not ta else bsa.dds(L, B.transpose(-1, -2).contiguous(),
                                                                                   P, trans_a=True)
        assert torch.all(D == 0)
