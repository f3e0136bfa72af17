"""GPU parity of the dense additive masks (attention mask [Nq, Nk] shared by
batch and heads, key-padding mask [Z, Nk]) in the softmax, the fused
attention and the backward, against the oracle with the same masks.

Masks hold N(0, 1) biases with about a tenth of the entries at -inf, one
query row and one batch element's keys beyond a length fully at -inf.
Tolerances as for the unmasked operators (TOL per dtype; gradients scaled
by max(1, max |reference|)).
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

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _qkv(shapes, seed, dt):
    g = torch.Generator("cpu").manual_seed(seed)
    return [torch.randn(s, generator=g).to(DT[dt]) for s in shapes]


def _masks(Z, Nq, Nk, seed, which="both"):
    """(attn_mask, key_padding_mask) as float32 CPU tensors (or None)."""
    g = torch.Generator("cpu").manual_seed(seed)
    am = torch.randn((Nq, Nk), generator=g)
    am[torch.rand((Nq, Nk), generator=g) < 0.1] = -float("inf")
    am[3, :] = -float("inf")                      # one query row sees nothing
    kp = torch.randn((Z, Nk), generator=g) * 0.5
    kp[Z - 1, Nk - Nk // 3:] = -float("inf")      # key padding of the last batch element
    return (am if which in ("both", "attn") else None), (kp if which in ("both", "kp") else None)


def _dev(m):
    return None if m is None else to_dev(m)


@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("which", ["attn", "kp", "both"])
def test_softmax_masked(b, causal, which):
    H, nb, Z = 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, 300 + b, force_diagonal=True)
    lay[1, 2, :] = 0
    nnz = int(lay.sum())
    announce("softmax masked", b, causal, which)
    g = torch.Generator("cpu").manual_seed(301)
    S = torch.randn((Z, nnz, b, b), generator=g) * 3
    am, kp = _masks(Z, nb * b, nb * b, 302 + b, which)
    L = bsa.Layout(torch.from_numpy(lay), b)
    P = bsa.softmax(L, to_dev(S), 0.6, causal, attn_mask=_dev(am), key_padding_mask=_dev(kp))
    ref = oracle.softmax(S, lay, b, 0.6, causal, am, kp)
    assert not torch.isnan(P).any()
    assert max_abs(f64(P), ref) <= TOL["f32"]


def test_softmax_masked_nonsquare_long_rows():
    """A non-square layout whose rows exceed the register cache (the re-read
    path), with both masks."""
    lay = W.small_random_layout(2, 3, 150, 0.6, 303)
    nnz = int(lay.sum())
    announce("softmax masked non-square long rows")
    g = torch.Generator("cpu").manual_seed(304)
    S = torch.randn((2, nnz, 16, 16), generator=g)
    am, kp = _masks(2, 3 * 16, 150 * 16, 305)
    L = bsa.Layout(torch.from_numpy(lay), 16)
    P = bsa.softmax(L, to_dev(S), 0.5, attn_mask=_dev(am), key_padding_mask=_dev(kp))
    assert max_abs(f64(P), oracle.softmax(S, lay, 16, 0.5, False, am, kp)) <= TOL["f32"]


ATTN_CASES = [(b, d, dt, causal) for b in (16, 32, 64, 128) for d in (64, 128) for dt in ("f32", "bf16", "f16")
              for causal in (False, True)]


@pytest.mark.parametrize("b,d,dt,causal", ATTN_CASES)
def test_attention_masked(b, d, dt, causal):
    H, nb, Z = 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, 310 + b + d, force_diagonal=True)
    lay[1, 2, :] = 0
    announce("attention masked", b, d, dt, causal)
    q, k, v = _qkv([(Z, H, nb * b, d)] * 3, 311 + b, dt)
    am, kp = _masks(Z, nb * b, nb * b, 312 + d)
    scale = 1.0 / np.sqrt(d)
    L = bsa.Layout(torch.from_numpy(lay), b)
    O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), scale, causal, attn_mask=_dev(am),
                      key_padding_mask=_dev(kp))
    assert O.dtype == q.dtype and not torch.isnan(O).any()
    ref = oracle.attention_dense(q, k, v, lay, b, scale, causal, am, kp)
    assert max_abs(f64(O), ref) <= TOL[dt]


@pytest.mark.parametrize("which", ["attn", "kp"])
@pytest.mark.parametrize("b", [16, 64])
def test_attention_one_mask_nonsquare(which, b):
    H, nbr, nbc, Z, d = 2, 3, 5, 2, 64
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 320 + b)
    lay[:, :, 0] = 1
    announce("attention one mask non-square", which, b)
    g = torch.Generator("cpu").manual_seed(321)
    q = torch.randn((Z, H, nbr * b, d), generator=g)
    k, v = (torch.randn((Z, H, nbc * b, d), generator=g) for _ in range(2))
    am, kp = _masks(Z, nbr * b, nbc * b, 322, which)
    L = bsa.Layout(torch.from_numpy(lay), b)
    O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), 0.125, attn_mask=_dev(am), key_padding_mask=_dev(kp))
    assert max_abs(f64(O), oracle.attention_dense(q, k, v, lay, b, 0.125, False, am, kp)) <= TOL["f32"]


@pytest.mark.parametrize("b", [16, 32, 64, 128])
def test_zero_masks_give_the_unmasked_bits_fp32(b):
    """fp32: s * 1 + log2(e) * 0 is s, so zero masks must reproduce the
    unmasked fused output bit for bit when both launches deal the rows the
    same way (one key group per row: a batch large enough that no row is
    split; the masked variant allows fewer key groups)."""
    H, nb, Z, d = 2, 4, 256, 64
    lay = W.small_random_layout(H, nb, nb, 0.5, 330 + b, force_diagonal=True)
    announce("zero masks fp32", b)
    q, k, v = (to_dev(t) for t in _qkv([(Z, H, nb * b, d)] * 3, 331, "f32"))
    L = bsa.Layout(torch.from_numpy(lay), b)
    am = torch.zeros((nb * b, nb * b), device="cuda")
    kp = torch.zeros((Z, nb * b), device="cuda")
    for causal in (False, True):
        O0 = bsa.attention(L, q, k, v, 0.125, causal)
        O1 = bsa.attention(L, q, k, v, 0.125, causal, attn_mask=am, key_padding_mask=kp)
        assert torch.equal(O0, O1)


def test_key_padding_full_size_causal_b64_sampled_rows():
    """causal_b64 at full size with per-sequence lengths as a key-padding
    mask; sampled block rows (including rows past a sequence's length,
    which still see their unpadded keys)."""
    w = W.WORKLOADS[1]
    lay = W.make_layout(w)
    q, k, v = W.make_qkv(w)
    N = w.nb * w.block
    lens = np.random.default_rng(340).integers(N // 4, N + 1, size=w.Z)
    kp = torch.zeros((w.Z, N))
    for z, n in enumerate(lens):
        kp[z, int(n):] = -float("inf")
    announce("key padding full size", w.name)
    L = bsa.Layout(torch.from_numpy(lay), w.block)
    O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), w.scale, w.causal, key_padding_mask=to_dev(kp))
    rows = [(0, 0, w.nb - 1), (w.Z - 1, w.H - 1, w.nb // 2), (w.Z // 2, 3, 5), (1, 7, w.nb - 3)]
    ref = oracle.attention_rows(q, k, v, lay, w.block, w.scale, w.causal, rows, kp_mask=kp)
    for n, (z, h, r) in enumerate(rows):
        got = f64(O[z, h, r * w.block:(r + 1) * w.block])
        assert max_abs(got, ref[n]) <= TOL["f32"], (z, h, r)


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("b", [16, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_backward_masked(dt, b, causal):
    H, nb, Z, d = 2, 4, 2, 64
    lay = W.small_random_layout(H, nb, nb, 0.5, 350 + b, force_diagonal=True)
    announce("attention_backward masked", dt, b, causal)
    q, k, v, do = _qkv([(Z, H, nb * b, d)] * 4, 351, dt)
    am, kp = _masks(Z, nb * b, nb * b, 352)
    L = bsa.Layout(torch.from_numpy(lay), b)
    grads = bsa.attention_backward(L, to_dev(q), to_dev(k), to_dev(v), to_dev(do), 0.125, causal,
                                   attn_mask=_dev(am), key_padding_mask=_dev(kp))
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, 0.125, causal, am, kp)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        tol = TOL[dt] * (1.0 if dt == "f32" else max(1.0, float(np.abs(ref).max())))
        assert max_abs(f64(got), ref) <= tol, name


def test_autograd_with_masks():
    b, d, H, nb, Z = 32, 64, 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, 360, force_diagonal=True)
    announce("autograd masked")
    q, k, v, do = _qkv([(Z, H, nb * b, d)] * 4, 361, "f32")
    am, kp = _masks(Z, nb * b, nb * b, 362)
    L = bsa.Layout(torch.from_numpy(lay), b)
    qd, kd, vd = (to_dev(t).requires_grad_(True) for t in (q, k, v))
    o = bsa.attention_autograd(L, qd, kd, vd, 0.125, True, attn_mask=_dev(am), key_padding_mask=_dev(kp))
    assert max_abs(f64(o.detach()), oracle.attention_dense(q, k, v, lay, b, 0.125, True, am, kp)) <= TOL["f32"]
    o.backward(to_dev(do))
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, 0.125, True, am, kp)
    for got, ref in zip((qd.grad, kd.grad, vd.grad), refs):
        assert max_abs(f64(got), ref) <= TOL["f32"]


def test_mask_argument_errors():
    """Wrong mask shape or dtype is refused by the binding; a misaligned mask
    pointer by the library (before anything is launched)."""
    lay = np.ones((1, 2, 2), np.uint8)
    announce("mask argument errors")
    L = bsa.Layout(torch.from_numpy(lay), 16)
    q = torch.zeros((1, 1, 32, 64), device="cuda")
    with pytest.raises(ValueError):
        bsa.attention(L, q, q, q, attn_mask=torch.zeros((32, 16), device="cuda"))
    with pytest.raises(ValueError):
        bsa.attention(L, q, q, q, key_padding_mask=torch.zeros((1, 32), device="cuda", dtype=torch.float16))
    buf = torch.zeros(32 * 32 + 1, device="cuda")
    o = torch.empty_like(q)
    p = lambda t: C.c_void_p(t.data_ptr())
    rc = _lib.lib().bs_attention_masked(L.handle, p(q), p(q), p(q), p(o), 1, 64, 0.125, 0,
                                        C.c_void_p(buf.data_ptr() + 4), None, _lib.BS_F32, None)
    assert rc == _lib.BS_ERR_INVALID_ARG
