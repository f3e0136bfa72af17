"""GPU parity of the fused attention with fp8 score operands (BS_F8E4M3):
Q and K are OCP FP8 E4M3, V and O bfloat16.

The oracle runs in float64 on the fp8 values of Q and K (exact in float64)
and the bf16 V. Bar: the bf16 one, 2e-2 max-abs. Derivation: the products
of two E4M3 values are exact in float32 and the fp32 sums of d = 128 of
them carry a relative error of about 1e-6 (scores below 60 in size move by
under 1e-4, so P moves by under 1e-4 relative); after that the path is the
bf16 one (P rounded RNE to bf16, unit roundoff 2^-9, with the row sum over
the same rounded values, and O rounded once), whose bar is 2e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, WORKERS, announce, f64, max_abs, pool_map, to_dev

import block_sparse_matmul_amd as bsa
from block_sparse_matmul_amd import _lib

pytestmark = pytest.mark.gpu

F8 = torch.float8_e4m3fn
LSE_TOL = 4e-3  # as bf16: the row sum adds the bf16-rounded P (|d log l| <= 2^-9)


def _inputs(Z, H, N, d, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    q, k, v = [torch.randn((Z, H, N, d), generator=g) for _ in range(3)]
    return q.to(F8), k.to(F8), v.to(torch.bfloat16)


@pytest.mark.parametrize("b", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_attention_matches_oracle(b, causal):
    H, nb, Z, d = 2, 4, 2, 128
    lay = W.small_random_layout(H, nb, nb, 0.5, 800 + b, force_diagonal=True)
    lay[1, 2, :] = 0  # an empty block row
    announce("fp8 attention", b, causal)
    q, k, v = _inputs(Z, H, nb * b, d, 801 + b)
    L = bsa.Layout(torch.from_numpy(lay), b)
    qd = to_dev(q)
    o = bsa.attention(L, qd, to_dev(k), to_dev(v), 0.125, causal, out=torch.full(q.shape, float("nan"),
                                                                                 dtype=torch.bfloat16,
                                                                                 device="cuda"))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16 and bool(torch.isfinite(o).all())
    ref = oracle.attention_dense(q, k, v, lay, b, 0.125, causal)
    assert max_abs(f64(o), ref) <= TOL["bf16"]
    # route (ii) agrees too
    assert max_abs(f64(o), oracle.attention_blocks(q, k, v, lay, b, 0.125, causal)) <= TOL["bf16"]


@pytest.mark.parametrize("b", [64, 128])
def test_fp8_attention_lse_and_masks(b):
    H, nb, Z, d = 2, 3, 2, 128
    lay = W.small_random_layout(H, nb, nb, 0.6, 810 + b, force_diagonal=True)
    announce("fp8 attention lse + masks", b)
    q, k, v = _inputs(Z, H, nb * b, d, 811 + b)
    g = torch.Generator("cpu").manual_seed(812)
    am = torch.randn((nb * b, nb * b), generator=g)
    am[torch.rand(am.shape, generator=g) < 0.1] = float("-inf")
    kp = 0.5 * torch.randn((Z, nb * b), generator=g)
    kp[1, 2 * b:] = float("-inf")
    L = bsa.Layout(torch.from_numpy(lay), b)
    o, lse = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), 0.125, attn_mask=to_dev(am),
                           key_padding_mask=to_dev(kp), return_lse=True)
    torch.cuda.synchronize()
    ref = oracle.attention_dense(q, k, v, lay, b, 0.125, False, am, kp)
    assert max_abs(f64(o), ref) <= TOL["bf16"]
    ref_lse = oracle.attention_lse(q, k, lay, b, 0.125, False, am, kp)
    got = f64(lse)
    inf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got), inf)
    assert float(np.abs(got[~inf] - ref_lse[~inf]).max()) <= LSE_TOL


def test_fp8_full_size_random_b128_every_row():
    """random_b128_bf16's layout and shape with Q and K rounded to fp8:
    every block row against the oracle's per-block route."""
    w = W.workload("random_b128_bf16")
    announce("fp8 full size", w.name)
    lay = W.make_layout(w)
    q, k, v = W.make_qkv(w)
    q8, k8 = q.float().to(F8), k.float().to(F8)
    L = bsa.Layout(torch.from_numpy(lay), w.block)
    o = bsa.attention(L, to_dev(q8), to_dev(k8), to_dev(v), w.scale,
                      out=torch.full(v.shape, float("nan"), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    Q, K, V = oracle._f64(q8), oracle._f64(k8), oracle._f64(v)
    rows = [(z, h, r) for z in range(w.Z) for h in range(w.H) for r in range(w.nb)]
    chunks = [rows[i::WORKERS] for i in range(WORKERS)]
    res = pool_map(lambda c: [oracle.attention_blockrow(Q, K, V, lay, w.block, w.scale, False, *x) for x in c],
                    chunks)
    got = f64(o)
    b = w.block
    worst = 0.0
    for chunk, outs in zip(chunks, res):
        for (z, h, r), ref in zip(chunk, outs):
            worst = max(worst, max_abs(got[z, h, r * b:(r + 1) * b], ref))
    assert worst <= TOL["bf16"], worst


def test_fp8_rejected_where_not_supported():
    announce("fp8 rejections")
    lay = np.ones((1, 2, 2), np.uint8)
    q, k, v = _inputs(1, 1, 128, 64, 820)  # d = 64: no fp8 kernel
    L = bsa.Layout(torch.from_numpy(lay), 64)
    with pytest.raises(bsa.BsError) as e:
        bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), 0.125)
    assert e.value.code == _lib.BS_ERR_UNSUPPORTED
    L16 = bsa.Layout(torch.from_numpy(np.ones((1, 8, 8), np.uint8)), 16)
    q, k, v = _inputs(1, 1, 128, 128, 821)  # 16-blocks: no fp8 kernel
    with pytest.raises(bsa.BsError) as e:
        bsa.attention(L16, to_dev(q), to_dev(k), to_dev(v), 0.125)
    assert e.value.code == _lib.BS_ERR_UNSUPPORTED
    with pytest.raises(bsa.BsError) as e:  # the unfused products take no fp8
        bsa.sdd(L16, to_dev(q), to_dev(k))
    assert e.value.code == _lib.BS_ERR_UNSUPPORTED
