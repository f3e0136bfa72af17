"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times, checked on sampled outputs the oracle computes one by
one (block rows of O, blocks of S, rows of P, block columns of the DDS)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (TOL, announce, f64, max_abs, oracle_block_sdd, oracle_row_softmax, sample_rows,
                         to_dev)

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


@pytest.mark.parametrize("idx", range(5), ids=[w.name for w in W.WORKLOADS])
def test_fused_attention_full_size_sampled_rows(idx):
    w = W.WORKLOADS[idx]
    announce("fused full", w.name)
    lay, q, k, v, L = _setup(w)
    assert L.nnz == int(lay.sum())
    O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), w.scale, w.causal)
    torch.cuda.synchronize()
    rows = sample_rows(lay, w.Z, 6, seed=idx)
    ref = oracle.attention_rows(q, k, v, lay, w.block, w.scale, w.causal, rows)
    b = w.block
    for n, (z, h, r) in enumerate(rows):
        got = f64(O[z, h, r * b:(r + 1) * b])
        assert max_abs(got, ref[n]) <= TOL[w.dtype], (z, h, r)
    assert not torch.isnan(O).any()


@pytest.mark.parametrize("idx", range(5), ids=[w.name for w in W.WORKLOADS])
def test_unfused_chain_full_size_sampled(idx):
    w = W.WORKLOADS[idx]
    announce("unfused full", w.name)
    lay, q, k, v, L = _setup(w)
    lut = oracle.lut_from_layout(lay)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    S = bsa.sdd(L, qd, kd)
    rng = np.random.default_rng(100 + idx)
    blocks = [(int(rng.integers(w.Z)), int(rng.integers(L.nnz))) for _ in range(8)]
    blocks.append((w.Z - 1, L.nnz - 1))
    for z, kk in blocks:
        ref = oracle_block_sdd(q, k, lay, lut, w.block, z, kk)
        assert max_abs(f64(S[z, kk]), ref) <= TOL["f32"], (z, kk)
    P = bsa.softmax(L, S, w.scale, w.causal, inplace=True)
    O = bsa.dsd(L, P, vd)
    torch.cuda.synchronize()
    rows = sample_rows(lay, w.Z, 3, seed=idx)
    b = w.block
    for z, h, r in rows[:3]:
        ks = range(lut["row_ptr"][h * w.nb + r], lut["row_ptr"][h * w.nb + r + 1])
        if len(ks) == 0:
            continue
        ref = oracle_row_softmax(q, k, lay, b, w.scale, w.causal, z, h, r)
        got = np.stack([f64(P[z, kk]) for kk in ks])
        assert max_abs(got, ref) <= TOL["f32"], (z, h, r)
    ref_o = oracle.attention_rows(q, k, v, lay, b, w.scale, w.causal, rows)
    for n, (z, h, r) in enumerate(rows):
        assert max_abs(f64(O[z, h, r * b:(r + 1) * b]), ref_o[n]) <= TOL[w.dtype], (z, h, r)


def test_dds_full_size_strided_sampled_columns():
    w = W.workload("strided_acsr_b32")
    announce("dds full", w.name)
    lay = W.make_layout(w)
    L = bsa.Layout.acsr(W.make_acsr(w), w.H, w.nb, w.nb, w.block)
    A, S = W.make_dds_operands(w, L.nnz)
    C = bsa.dds(L, to_dev(A), to_dev(S))
    torch.cuda.synchronize()
    lut = oracle.lut_from_layout(lay)
    b, nb = w.block, w.nb
    rng = np.random.default_rng(5)
    cols = {(0, 0), (w.H - 1, nb - 1)} | {(int(rng.integers(w.H)), int(rng.integers(nb))) for _ in range(6)}
    for h, c in sorted(cols):
        e0, e1 = lut["col_ptr"][h * nb + c], lut["col_ptr"][h * nb + c + 1]
        sub = np.zeros((1, nb, nb), np.uint8)
        sub[0, :, c] = lay[h, :, c]
        S_sub = S[:, torch.from_numpy(lut["blk_id"][e0:e1].astype(np.int64))]
        ref = oracle.dds(A[:, h:h + 1], S_sub, sub, b)[0, 0, :, c * b:(c + 1) * b]
        assert max_abs(f64(C[0, h, :, c * b:(c + 1) * b]), ref) <= TOL["f32"], (h, c)
