"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times.

Every output tensor is first filled with NaN, so that an element the kernels
never write (a row the scheduler skipped, or wrote to the wrong place) shows
up. Then:
  * the fused attention: every block row of O against the oracle (dense
    masked rows, route (i), for the fp32 workloads; the per-block route
    (ii) for random_b128_bf16, which only touches stored blocks);
  * the unfused chain SDD -> softmax -> DSD: every block of S and P against
    the oracle for the fp32 workloads, every block row of O for all five
    (S and P of random_b128_bf16, 8.8 GB each, are checked finite on the
    device and compared on sampled blocks and rows);
  * the standalone DDS of the strided workload: every block column.
The oracle's rows are computed in a thread pool (numpy releases the
interpreter lock in its kernels), with one BLAS thread per worker.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (TOL, WORKERS, announce, f64, max_abs, oracle_block_sdd, oracle_row_softmax, pool_map,
                         sample_rows, to_dev)

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_matmul_amd")

def _setup(w):
    lay = W.make_layout(w)
    q, k, v = W.make_qkv(w)
    if w.pattern == "strided_acsr":
        L = bsa.Layout.acsr(W.make_acsr(w), w.H, w.nb, w.nb, w.block)
    else:
        L = bsa.Layout(torch.from_numpy(lay), w.block)
    return lay, q, k, v, L


def _nan_like(t):
    return torch.full_like(t, float("nan"))


def oracle_all_rows(w, lay, q, k, v):
    """The oracle's O for every block row of the workload, [Z, H, N, d]
    float64."""
    Q, K, V = oracle._f64(q), oracle._f64(k), oracle._f64(v)
    rows = [(z, h, r) for z in range(w.Z) for h in range(w.H) for r in range(w.nb)]
    chunks = [rows[i::WORKERS] for i in range(WORKERS)]
    b = w.block
    if w.dtype == "bf16":
        def run(chunk):
            return [oracle.attention_blockrow(Q, K, V, lay, b, w.scale, w.causal, z, h, r) for z, h, r in chunk]
    else:
        def run(chunk):
            return list(oracle.attention_rows(Q, K, V, lay, b, w.scale, w.causal, chunk))
    out = np.zeros(Q.shape[:3] + (V.shape[3],))
    for chunk, res in zip(chunks, pool_map(run, chunks)):
        for (z, h, r), o in zip(chunk, res):
            out[z, h, r * b:(r + 1) * b] = o
    return out


_REF = {}


def _ref_o(w, lay, q, k, v):
    if w.name not in _REF:
        _REF[w.name] = oracle_all_rows(w, lay, q, k, v)
    return _REF[w.name]


@pytest.mark.parametrize("idx", range(5), ids=[w.name for w in W.WORKLOADS])
def test_fused_attention_full_size_every_row(idx):
    w = W.WORKLOADS[idx]
    announce("fused full, every row", w.name)
    lay, q, k, v, L = _setup(w)
    assert L.nnz == int(lay.sum())
    qd = to_dev(q)
    O = bsa.attention(L, qd, to_dev(k), to_dev(v), w.scale, w.causal, out=_nan_like(qd))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all()), "unwritten or non-finite output"
    ref = _ref_o(w, lay, q, k, v)
    got = f64(O)
    b = w.block
    err = np.abs(got - ref).reshape(w.Z, w.H, w.nb, b * w.d).max(axis=3)
    worst = np.unravel_index(int(np.argmax(err)), err.shape)
    assert err.max() <= TOL[w.dtype], ("block row", worst, float(err.max()))


@pytest.mark.parametrize("idx", range(5), ids=[w.name for w in W.WORKLOADS])
def test_unfused_chain_full_size(idx):
    w = W.WORKLOADS[idx]
    announce("unfused full", w.name)
    lay, q, k, v, L = _setup(w)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    S = torch.full((w.Z, L.nnz, w.block, w.block), float("nan"), device="cuda")
    bsa.sdd(L, qd, kd, out=S)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(S).all()), "unwritten S"
    full = w.dtype == "f32"
    lut = oracle.lut_from_layout(lay)
    if full:
        S_ref = oracle.sdd(q, k, lay, w.block)
        assert max_abs(f64(S), S_ref) <= TOL["f32"]
    else:
        rng = np.random.default_rng(100 + idx)
        blocks = [(int(rng.integers(w.Z)), int(rng.integers(L.nnz))) for _ in range(24)]
        blocks.append((w.Z - 1, L.nnz - 1))
        for z, kk in blocks:
            ref = oracle_block_sdd(q, k, lay, lut, w.block, z, kk)
            assert max_abs(f64(S[z, kk]), ref) <= TOL["f32"], (z, kk)
    P = torch.full_like(S, float("nan"))
    bsa.softmax(L, S, w.scale, w.causal, out=P)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(P).all()), "unwritten P"
    if full:
        P_ref = oracle.softmax(S_ref, lay, w.block, w.scale, w.causal)
        assert max_abs(f64(P), P_ref) <= TOL["f32"]
        del S_ref, P_ref
    else:
        for z, h, r in sample_rows(lay, w.Z, 6, seed=idx):
            ks = range(lut["row_ptr"][h * w.nb + r], lut["row_ptr"][h * w.nb + r + 1])
            if len(ks) == 0:
                continue
            ref = oracle_row_softmax(q, k, lay, w.block, w.scale, w.causal, z, h, r)
            got = np.stack([f64(P[z, kk]) for kk in ks])
            assert max_abs(got, ref) <= TOL["f32"], (z, h, r)
    del S
    O = bsa.dsd(L, P, vd, out=_nan_like(qd))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all()), "unwritten O"
    ref_o = _ref_o(w, lay, q, k, v)
    assert max_abs(f64(O), ref_o) <= TOL[w.dtype]


def test_dds_full_size_strided_every_column():
    w = W.workload("strided_acsr_b32")
    announce("dds full, every column", w.name)
    lay = W.make_layout(w)
    L = bsa.Layout.acsr(W.make_acsr(w), w.H, w.nb, w.nb, w.block)
    A, S = W.make_dds_operands(w, L.nnz)
    Ad = to_dev(A)
    C = torch.full((w.Z, w.H, w.dds_m, w.N), float("nan"), device="cuda")
    bsa.dds(L, Ad, to_dev(S), out=C)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(C).all()), "unwritten C"
    ref = oracle.dds(A, S, lay, w.block)
    err = np.abs(f64(C) - ref).reshape(w.Z, w.H, w.dds_m, w.nb, w.block).max(axis=(2, 4))
    worst = np.unravel_index(int(np.argmax(err)), err.shape)
    assert err.max() <= TOL["f32"], ("block column", worst, float(err.max()))
