"""Fused attention on ACSR layouts (SPLAT abstract: the affine-compressed
sparse-row format). When every term has slope 1 and covers every row, the
fused kernel computes each row's columns from one sorted set of relative
offsets instead of reading the column table; the order of the blocks is the
same ascending order, so the output must equal, bit for bit, the output for
the same pattern built from a dense layout. Other ACSR layouts keep the
tables. Parity against the oracle as for every layout. These tests keep the K/V
sharing across rows off (its kernel has tests of its own) except where
named.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, announce, f64, max_abs, to_dev

import block_sparse_matmul_amd as bsa

pytestmark = pytest.mark.gpu


def _qkv(Z, H, N, d, seed, dt="f32"):
    g = torch.Generator("cpu").manual_seed(seed)
    out = [torch.randn((Z, H, N, d), generator=g) for _ in range(3)]
    return [t.to(torch.bfloat16) for t in out] if dt == "bf16" else out


# (terms, nb): band-and-strided like the strided workload; overlapping terms
# with a negative offset beyond the grid, stride 0 and a negative stride;
# terms whose offsets leave some rows empty
SLOPE1_CASES = [
    ([(0, 12, 1, -3, 1, 4), (0, 12, 1, -12, 4, 4)], 12),
    ([(0, 9, 1, -20, 1, 30), (-5, 20, 1, 2, 0, 7), (0, 9, 1, 3, -2, 3)], 9),
    ([(0, 8, 1, 5, 1, 2)], 8),
]


@pytest.mark.parametrize("case", range(len(SLOPE1_CASES)))
@pytest.mark.parametrize("b", [16, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_slope1_acsr_attention_equals_dense_layout_and_oracle(case, b, causal):
    terms, nb = SLOPE1_CASES[case]
    H, Z, d = 2, 2, 64
    lay = oracle.acsr_expand(terms, H, nb, nb)
    announce("acsr attention", case, b, causal)
    q, k, v = _qkv(Z, H, nb * b, d, 30 + case)
    La = bsa.Layout.acsr(terms, H, nb, nb, b)
    La.set_kv_share(False)
    Ld = bsa.Layout(torch.from_numpy(lay), b)
    Oa = bsa.attention(La, to_dev(q), to_dev(k), to_dev(v), 0.125, causal)
    Od = bsa.attention(Ld, to_dev(q), to_dev(k), to_dev(v), 0.125, causal)
    assert torch.equal(Oa, Od)
    assert max_abs(f64(Oa), oracle.attention_dense(q, k, v, lay, b, 0.125, causal)) <= TOL["f32"]


def test_non_slope1_acsr_keeps_the_tables():
    terms = [(0, 10, 2, -4, 1, 3), (0, 10, 1, 0, 1, 1)]  # slope 2: no common offset set
    H, Z, nb, b, d = 1, 1, 10, 32, 64
    lay = oracle.acsr_expand(terms, H, nb, 2 * nb)
    announce("acsr slope 2")
    g = torch.Generator("cpu").manual_seed(40)
    q = torch.randn((Z, H, nb * b, d), generator=g)
    k, v = (torch.randn((Z, H, 2 * nb * b, d), generator=g) for _ in range(2))
    L = bsa.Layout.acsr(terms, H, nb, 2 * nb, b)
    O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), 0.125)
    assert max_abs(f64(O), oracle.attention_dense(q, k, v, lay, b, 0.125)) <= TOL["f32"]


def test_strided_workload_acsr_path_bit_equal_to_table_path():
    """The strided workload at full size: the fused kernel from 76 column
    offsets gives the same bits as from its 180,736-entry column table; so
    does the kernel that shares K/V across rows (one key group per row, as
    the table path runs this workload: the same blocks in the same order
    with the same arithmetic)."""
    w = W.workload("strided_acsr_b32")
    announce("acsr strided full size")
    q, k, v = (to_dev(t) for t in W.make_qkv(w))
    La = bsa.Layout.acsr(W.make_acsr(w), w.H, w.nb, w.nb, w.block)
    Ld = bsa.Layout(torch.from_numpy(W.make_layout(w)), w.block)
    assert La.kv_share() == (2, 4)
    La.set_kv_share(True)
    Os = bsa.attention(La, q, k, v, w.scale, w.causal)
    La.set_kv_share(False)
    Oa = bsa.attention(La, q, k, v, w.scale, w.causal)
    Od = bsa.attention(Ld, q, k, v, w.scale, w.causal)
    assert torch.equal(Oa, Od)
    assert torch.equal(Os, Od)


@pytest.mark.parametrize("b", [16, 64])
def test_slope1_acsr_with_masks_lse_and_fused_backward(b):
    """The computed-column path with a key-padding mask and the row
    log-sum-exp: the same bits as the dense layout's table path, and the
    fused backward (which walks the tables) against the oracle."""
    terms, nb = SLOPE1_CASES[0]
    H, Z, d = 2, 2, 64
    N = nb * b
    lay = oracle.acsr_expand(terms, H, nb, nb)
    announce("acsr masked lse backward", b)
    q, k, v = _qkv(Z, H, N, d, 45)
    g = torch.Generator("cpu").manual_seed(46)
    kp = torch.randn((Z, N), generator=g)
    kp[1, N // 2:] = -float("inf")
    do = torch.randn((Z, H, N, d), generator=g)
    La = bsa.Layout.acsr(terms, H, nb, nb, b)
    La.set_kv_share(False)
    Ld = bsa.Layout(torch.from_numpy(lay), b)
    qd, kd, vd, kpd = to_dev(q), to_dev(k), to_dev(v), to_dev(kp)
    Oa, la = bsa.attention(La, qd, kd, vd, 0.125, True, key_padding_mask=kpd, return_lse=True)
    Od, ld = bsa.attention(Ld, qd, kd, vd, 0.125, True, key_padding_mask=kpd, return_lse=True)
    assert torch.equal(Oa, Od) and torch.equal(la, ld)
    assert max_abs(f64(Oa), oracle.attention_dense(q, k, v, lay, b, 0.125, True, kp_mask=kp)) <= TOL["f32"]
    grads = bsa.attention_backward_fused(La, qd, kd, vd, Oa, la, to_dev(do), 0.125, True, key_padding_mask=kpd)
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, 0.125, True, kp_mask=kp)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        assert max_abs(f64(got), ref) <= TOL["f32"], name
