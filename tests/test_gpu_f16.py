"""GPU parity with IEEE fp16 dense operands, against the oracle on the same
fp16-rounded inputs (converted exactly to float64).

Every mode takes fp16 the way it takes bf16: products on the 16-bit matrix
cores with fp32 accumulation, fp32 values that feed a product (P, S, dS)
rounded to fp16 (RNE), results rounded once. The SDD's output is fp32 from
exact fp16 products, so it keeps the fp32 bar; everything with an fp16
output or an fp16-rounded factor takes TOL["f16"] (its derivation is in
gpu_helpers). Cases span every block size, both head sizes, causal and not,
the generic kernels (other K / Nd), and the 32-rows-per-wave fused kernel's
key-group schedules.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, announce, f64, max_abs, to_dev

import block_sparse_matmul_amd as bsa
from block_sparse_matmul_amd import _lib

pytestmark = pytest.mark.gpu


def _h(shapes, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return [torch.randn(shp, generator=g, dtype=torch.float32).to(torch.float16) for shp in shapes]


def _grad_tol(ref):
    return TOL["f16"] * max(1.0, float(np.abs(ref).max()))


@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("K", [64, 128, 48])
def test_sdd_f16(b, K):
    H, nbr, nbc, Z = 2, 3, 4, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 200 + b + K)
    lay[0, 1, :] = 0
    announce("sdd f16", b, K)
    a, bb = _h([(Z, H, nbr * b, K), (Z, H, nbc * b, K)], 201)
    L = bsa.Layout(torch.from_numpy(lay), b)
    S = bsa.sdd(L, to_dev(a), to_dev(bb))
    assert S.dtype == torch.float32
    assert max_abs(f64(S), oracle.sdd(a, bb, lay, b)) <= TOL["f32"]


@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("Nd", [64, 128, 16])
def test_dsd_f16(b, Nd):
    H, nbr, nbc, Z = 2, 4, 3, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 210 + b + Nd)
    lay[1, 3, :] = 0
    nnz = int(lay.sum())
    announce("dsd f16", b, Nd)
    (Bm,) = _h([(Z, H, nbc * b, Nd)], 211)
    g = torch.Generator("cpu").manual_seed(212)
    P = torch.rand((Z, nnz, b, b), generator=g) / b
    L = bsa.Layout(torch.from_numpy(lay), b)
    Cm = bsa.dsd(L, to_dev(P), to_dev(Bm))
    assert Cm.dtype == torch.float16
    assert max_abs(f64(Cm), oracle.dsd(P, Bm, lay, b)) <= TOL["f16"]


@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("M", [32, 48, 80])
def test_dds_f16(b, M):
    H, nbr, nbc, Z = 2, 3, 5, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 220 + b + M)
    lay[0, :, 2] = 0
    nnz = int(lay.sum())
    announce("dds f16", b, M)
    (A,) = _h([(Z, H, M, nbr * b)], 221)
    g = torch.Generator("cpu").manual_seed(222)
    S = torch.rand((Z, nnz, b, b), generator=g) / b
    L = bsa.Layout(torch.from_numpy(lay), b)
    Cm = bsa.dds(L, to_dev(A), to_dev(S))
    assert Cm.dtype == torch.float16
    assert max_abs(f64(Cm), oracle.dds(A, S, lay, b)) <= TOL["f16"]


@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("Nd", [64, 128])
def test_dsd_t_f16(b, Nd):
    H, nbr, nbc, Z = 2, 3, 4, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 230 + b + Nd)
    lay[1, :, 2] = 0
    nnz = int(lay.sum())
    announce("dsd_t f16", b, Nd)
    (B,) = _h([(Z, H, nbr * b, Nd)], 231)
    g = torch.Generator("cpu").manual_seed(232)
    S = torch.rand((Z, nnz, b, b), generator=g) / b
    L = bsa.Layout(torch.from_numpy(lay), b)
    Cm = bsa.dsd_t(L, to_dev(S), to_dev(B))
    assert Cm.dtype == torch.float16
    assert max_abs(f64(Cm), oracle.dsd_t(S, B, lay, b)) <= TOL["f16"]


@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_f16(b, d, causal):
    H, nb, Z = 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, 240 + b + d, force_diagonal=True)
    lay[1, 2, :] = 0   # empty row -> zeros
    lay[0, 0, :] = 0
    lay[0, 0, 2] = 1   # causal hides this row completely -> zeros
    announce("attention f16", b, d, causal)
    q, k, v = _h([(Z, H, nb * b, d)] * 3, 241 + b)
    scale = 1.0 / np.sqrt(d)
    L = bsa.Layout(torch.from_numpy(lay), b)
    O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), scale, causal)
    assert O.dtype == torch.float16
    assert not torch.isnan(O).any()
    assert max_abs(f64(O), oracle.attention_dense(q, k, v, lay, b, scale, causal)) <= TOL["f16"]


F16_SWEEP = [(32, 1), (32, 256), (64, 1), (64, 80), (128, 1), (128, 256)]


@pytest.mark.parametrize("b,Z", F16_SWEEP)
@pytest.mark.parametrize("d", [64, 128])
def test_attention_f16_key_group_schedules(b, Z, d):
    """Blocks of 32 to 128 run on the 32-rows-per-wave kernel, its key-group
    count and row order following the batch size; sampled block rows."""
    H, nb = 2, 4
    lay = W.small_random_layout(H, nb, nb, 0.5, 250 + b, force_diagonal=True)
    announce("attention f16 sweep", b, Z, d)
    q, k, v = _h([(Z, H, nb * b, d)] * 3, 251)
    L = bsa.Layout(torch.from_numpy(lay), b)
    scale = 1.0 / np.sqrt(d)
    for causal in (False, True):
        O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), scale, causal)
        rows = [(0, 0, 0), (Z - 1, 1, nb - 1), (Z // 2, 0, 2), (Z // 3, 1, 1)]
        ref = oracle.attention_rows(q, k, v, lay, b, scale, causal, rows)
        for n, (z, h, r) in enumerate(rows):
            assert max_abs(f64(O[z, h, r * b:(r + 1) * b]), ref[n]) <= TOL["f16"], (z, h, r, causal)


def test_attention_f16_large_scores():
    """Scores of size 100 and more (q and k scaled by 8): e^score would
    overflow fp16 many times over. Scores are accumulated and exponentiated
    (after the running max is taken off) in fp32; only P, in [0, 1], and O
    are rounded to fp16, so nothing overflows."""
    b, d, H, nb, Z = 64, 64, 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, 260, force_diagonal=True)
    announce("attention f16 large scores")
    q, k, v = _h([(Z, H, nb * b, d)] * 3, 261)
    q = (q.float() * 8).to(torch.float16)
    k = (k.float() * 8).to(torch.float16)
    L = bsa.Layout(torch.from_numpy(lay), b)
    O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), 0.125, True)
    assert torch.isfinite(O).all()
    assert max_abs(f64(O), oracle.attention_dense(q, k, v, lay, b, 0.125, True)) <= TOL["f16"]


@pytest.mark.parametrize("b", [16, 64, 128])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_backward_f16(b, d, causal):
    H, nb, Z = 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, 270 + b + d, force_diagonal=True)
    lay[1, 2, :] = 0
    announce("attention_backward f16", b, d, causal)
    q, k, v, do = _h([(Z, H, nb * b, d)] * 4, 271 + b)
    scale = 1.0 / np.sqrt(d)
    L = bsa.Layout(torch.from_numpy(lay), b)
    grads = bsa.attention_backward(L, to_dev(q), to_dev(k), to_dev(v), to_dev(do), scale, causal)
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, scale, causal)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        assert got.dtype == torch.float16
        assert max_abs(f64(got), ref) <= _grad_tol(ref), name


def test_unfused_chain_f16_matches_fused():
    b, d, H, nb, Z = 32, 64, 3, 6, 2
    lay = W.small_random_layout(H, nb, nb, 0.4, 280, force_diagonal=True)
    announce("unfused chain f16")
    q, k, v = _h([(Z, H, nb * b, d)] * 3, 281)
    L = bsa.Layout(torch.from_numpy(lay), b)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    P = bsa.softmax(L, bsa.sdd(L, qd, kd), 0.125, causal=True)
    O1 = bsa.dsd(L, P, vd)
    O2 = bsa.attention(L, qd, kd, vd, 0.125, causal=True)
    ref = oracle.attention_dense(q, k, v, lay, b, 0.125, True)
    assert max_abs(f64(O1), ref) <= TOL["f16"]
    assert max_abs(f64(O2), ref) <= TOL["f16"]


def test_unknown_dtype_code_rejected():
    """A dtype code outside the header's enum is an invalid argument; nothing
    is launched."""
    lay = np.ones((1, 2, 2), np.uint8)
    announce("unknown dtype code")
    L = bsa.Layout(torch.from_numpy(lay), 16)
    a = torch.zeros((1, 1, 32, 64), device="cuda", dtype=torch.float16)
    s = torch.zeros((1, 4, 16, 16), device="cuda")
    ptr = lambda t: C.c_void_p(t.data_ptr())
    rc = _lib.lib().bs_sdd(L.handle, ptr(a), ptr(a), ptr(s), 1, 64, 4, None)
    assert rc == _lib.BS_ERR_INVALID_ARG
    # code 3 is BS_F8E4M3, defined but taken by the fused attention only
    rc = _lib.lib().bs_sdd(L.handle, ptr(a), ptr(a), ptr(s), 1, 64, _lib.BS_F8E4M3, None)
    assert rc == _lib.BS_ERR_UNSUPPORTED
