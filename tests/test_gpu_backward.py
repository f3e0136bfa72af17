"""GPU parity of the backward: softmax gradient, transposed DSD, the fused
attention backward entry point and the autograd wrapper, against the oracle.

Tolerances: float32 results to 1e-4 max-abs (the forward's bar); bf16
gradients (P and dS rounded to bf16 for the products, results rounded to
bf16) to 2e-2 of max(1, max |reference|) -- the forward's 2e-2 on outputs
of size about one, scaled to the size of the gradient.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, announce, f64, max_abs, pool_map, to_dev

import block_sparse_matmul_amd as bsa

pytestmark = pytest.mark.gpu


def _tensors(shapes, seed, dtype):
    g = torch.Generator("cpu").manual_seed(seed)
    out = []
    for shp in shapes:
        t = torch.randn(shp, generator=g, dtype=torch.float32)
        out.append(t.to(torch.bfloat16) if dtype == "bf16" else t)
    return out


def _grad_tol(dt, ref):
    return TOL["f32"] if dt == "f32" else 2e-2 * max(1.0, float(np.abs(ref).max()))


# ------------------------------------------------------------ softmax gradient

@pytest.mark.parametrize("b", [16, 32, 64, 128])
def test_softmax_backward(b):
    H, nb, Z = 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, 70 + b)
    lay[1, 2, :] = 0  # an empty row
    nnz = int(lay.sum())
    announce("softmax_backward", b)
    (S, G) = _tensors([(Z, nnz, b, b), (Z, nnz, b, b)], 71, "f32")
    L = bsa.Layout(torch.from_numpy(lay), b)
    P = bsa.softmax(L, to_dev(S), 0.6, causal=True)
    dS = bsa.softmax_backward(L, P, to_dev(G), 0.6)
    ref = oracle.softmax_backward(f64(P), G, lay, b, 0.6)
    assert max_abs(f64(dS), ref) <= TOL["f32"]
    # in place into dP
    dP = to_dev(G)
    out = bsa.softmax_backward(L, P, dP, 0.6, inplace=True)
    assert out.data_ptr() == dP.data_ptr()
    assert max_abs(f64(out), ref) <= TOL["f32"]


def test_softmax_backward_long_rows():
    # rows longer than the register cache (the re-read path): 300 blocks of 16
    lay = np.ones((1, 2, 300), np.uint8)
    announce("softmax_backward long rows")
    P, G = _tensors([(1, 600, 16, 16), (1, 600, 16, 16)], 72, "f32")
    P = torch.softmax(P.reshape(1, 2, 16, 300 * 16), -1)  # probability-like rows
    L = bsa.Layout(torch.from_numpy(lay), 16)
    Pd = to_dev(P.reshape(1, 2, 16, 300, 16).permute(0, 1, 3, 2, 4).reshape(1, 600, 16, 16))
    dS = bsa.softmax_backward(L, Pd, to_dev(G), 0.5)
    ref = oracle.softmax_backward(f64(Pd), G, lay, 16, 0.5)
    assert max_abs(f64(dS), ref) <= TOL["f32"]


# ------------------------------------------------------------ DSD^T

DSDT_CASES = [(b, n, dt) for b in (16, 32, 64, 128) for n, dt in ((64, "f32"), (128, "f32"), (64, "bf16"),
                                                                   (128, "bf16"))]


@pytest.mark.parametrize("b,Nd,dt", DSDT_CASES)
def test_dsd_t(b, Nd, dt):
    H, nbr, nbc, Z = 2, 3, 4, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 73 + b + Nd)
    lay[1, :, 2] = 0  # an empty block column: zero rows
    nnz = int(lay.sum())
    announce("dsd_t", b, Nd, dt)
    (B,) = _tensors([(Z, H, nbr * b, Nd)], 74, dt)
    g = torch.Generator("cpu").manual_seed(75)
    S = torch.rand((Z, nnz, b, b), generator=g) / b
    L = bsa.Layout(torch.from_numpy(lay), b)
    C = bsa.dsd_t(L, to_dev(S), to_dev(B))
    assert C.dtype == B.dtype and C.shape == (Z, H, nbc * b, Nd)
    assert max_abs(f64(C), oracle.dsd_t(S, B, lay, b)) <= TOL[dt]


@pytest.mark.parametrize("b", [16, 32, 64])
@pytest.mark.parametrize("Z", [1, 128, 256])
def test_dsd_t_batch_sweep_all_key_group_schedules(b, Z):
    """Columns split over 1, 2 or 4 key groups depending on the longest
    column against the work per CU; sampled batch entries against the oracle."""
    H, nb, Nd = 2, 4, 64
    lay = W.small_random_layout(H, nb, nb, 0.5, 76 + b, force_diagonal=True)
    nnz = int(lay.sum())
    announce("dsd_t batch sweep", b, Z)
    (B,) = _tensors([(Z, H, nb * b, Nd)], 77, "f32")
    g = torch.Generator("cpu").manual_seed(78)
    S = torch.rand((Z, nnz, b, b), generator=g) / b
    L = bsa.Layout(torch.from_numpy(lay), b)
    C = bsa.dsd_t(L, to_dev(S), to_dev(B))
    for z in sorted({0, Z // 3, Z // 2, Z - 1}):
        sl = slice(z, z + 1)
        assert max_abs(f64(C[sl]), oracle.dsd_t(S[sl], B[sl], lay, b)) <= TOL["f32"], z


# ------------------------------------------------------------ attention backward

BWD_CASES = [(b, d, dt, causal) for b in (16, 32, 64, 128) for d in (64, 128) for dt in ("f32", "bf16")
             for causal in (False, True)]


@pytest.mark.parametrize("b,d,dt,causal", BWD_CASES)
def test_attention_backward(b, d, dt, causal):
    H, nb, Z = 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, 80 + b + d, force_diagonal=True)
    lay[1, 2, :] = 0   # empty row: zero dq there, and no contribution to dk, dv
    announce("attention_backward", b, d, dt, causal)
    q, k, v, do = _tensors([(Z, H, nb * b, d)] * 4, 81 + b, dt)
    scale = 1.0 / np.sqrt(d)
    L = bsa.Layout(torch.from_numpy(lay), b)
    dq, dk, dv = bsa.attention_backward(L, to_dev(q), to_dev(k), to_dev(v), to_dev(do), scale, causal)
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, scale, causal)
    for name, got, ref in (("dq", dq, refs[0]), ("dk", dk, refs[1]), ("dv", dv, refs[2])):
        assert got.dtype == q.dtype
        assert max_abs(f64(got), ref) <= _grad_tol(dt, ref), name


def test_autograd_wrapper_matches_backward_entry_point_and_oracle():
    """The autograd function runs the forward with its row log-sum-exp and
    the fused backward: its gradients are that entry point's, bit for bit,
    and the oracle's."""
    b, d, H, nb, Z = 64, 64, 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, 90, force_diagonal=True)
    announce("attention autograd")
    q, k, v, do = _tensors([(Z, H, nb * b, d)] * 4, 91, "f32")
    L = bsa.Layout(torch.from_numpy(lay), b)
    qd, kd, vd = (to_dev(t).requires_grad_(True) for t in (q, k, v))
    o = bsa.attention_autograd(L, qd, kd, vd, 0.125, causal=True)
    assert max_abs(f64(o.detach()), oracle.attention_dense(q, k, v, lay, b, 0.125, True)) <= TOL["f32"]
    o.backward(to_dev(do))
    o2, lse = bsa.attention(L, qd.detach(), kd.detach(), vd.detach(), 0.125, True, return_lse=True)
    dq, dk, dv = bsa.attention_backward_fused(L, qd.detach(), kd.detach(), vd.detach(), o2, lse, to_dev(do), 0.125,
                                              True)
    for g_auto, g_direct in ((qd.grad, dq), (kd.grad, dk), (vd.grad, dv)):
        assert torch.equal(g_auto, g_direct)
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, 0.125, True)
    for got, ref in zip((qd.grad, kd.grad, vd.grad), refs):
        assert max_abs(f64(got), ref) <= TOL["f32"]


def test_attention_backward_full_size_causal_b64():
    """causal_b64 at full size (the launch configuration of the forward
    bench), every (batch, head) pair against the dense oracle gradient."""
    w = W.WORKLOADS[1]
    lay = W.make_layout(w)
    q, k, v = W.make_qkv(w)
    g = torch.Generator("cpu").manual_seed(92)
    do = torch.randn(q.shape, generator=g)
    announce("attention_backward full size", w.name)
    L = bsa.Layout(torch.from_numpy(lay), w.block)
    dq, dk, dv = bsa.attention_backward(L, to_dev(q), to_dev(k), to_dev(v), to_dev(do), w.scale, w.causal)
    got = {"dq": f64(dq), "dk": f64(dk), "dv": f64(dv)}

    def check(pair):
        z, h = pair
        sl = (slice(z, z + 1), slice(h, h + 1))
        refs = oracle.attention_backward_dense(q[sl], k[sl], v[sl], do[sl], lay[h:h + 1], w.block, w.scale, w.causal)
        return [(name, max_abs(got[name][sl], ref)) for name, ref in zip(("dq", "dk", "dv"), refs)]

    pairs = [(z, h) for z in range(w.Z) for h in range(w.H)]
    for pair, res in zip(pairs, pool_map(check, pairs)):
        for name, err in res:
            assert err <= TOL["f32"], (name, pair, err)
