"""GPU parity of the forward's row log-sum-exp and of the fused backward
(bs_attention_fwd, bs_attention_bwd) against the oracle.

lse bars: fp32 1e-4; 16-bit types sum the rounded P (relative error at
most the unit roundoff u of the type), so |d log l| <= u: bf16 u = 2^-9,
bar 4e-3; fp16 u = 2^-12, bar 1e-3. Gradient bars as for the composed
backward: fp32 1e-4 absolute, 16-bit TOL[dt] * max(1, max |reference|).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, announce, f64, max_abs, pool_map, to_dev

import block_sparse_matmul_amd as bsa

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
LSE_TOL = {"f32": 1e-4, "bf16": 4e-3, "f16": 1e-3}


def _t(shapes, seed, dt):
    g = torch.Generator("cpu").manual_seed(seed)
    return [torch.randn(s, generator=g).to(DT[dt]) for s in shapes]


def _grad_tol(dt, ref):
    return TOL["f32"] if dt == "f32" else TOL[dt] * max(1.0, float(np.abs(ref).max()))


def _lse_close(got, ref, tol):
    """Equal -inf where the row sees nothing, within tol elsewhere."""
    got = f64(got)
    inf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf)
    return float(np.abs(got[~inf] - ref[~inf]).max()) if (~inf).any() else 0.0


@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_lse(b, dt, causal):
    H, nb, Z, d = 2, 4, 2, 64
    lay = W.small_random_layout(H, nb, nb, 0.5, 400 + b, force_diagonal=True)
    lay[1, 2, :] = 0
    announce("forward lse", b, dt, causal)
    q, k, v = _t([(Z, H, nb * b, d)] * 3, 401, dt)
    L = bsa.Layout(torch.from_numpy(lay), b)
    o, lse = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), 0.125, causal, return_lse=True)
    o_plain = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), 0.125, causal)
    assert torch.equal(o, o_plain)
    assert _lse_close(lse, oracle.attention_lse(q, k, lay, b, 0.125, causal), LSE_TOL[dt]) <= LSE_TOL[dt]


@pytest.mark.parametrize("b", [16, 64])
def test_forward_lse_masked(b):
    H, nb, Z, d = 2, 4, 2, 64
    N = nb * b
    lay = W.small_random_layout(H, nb, nb, 0.5, 402 + b, force_diagonal=True)
    announce("forward lse masked", b)
    q, k, v = _t([(Z, H, N, d)] * 3, 403, "f32")
    g = torch.Generator("cpu").manual_seed(404)
    am = torch.randn((N, N), generator=g)
    am[3, :] = -float("inf")
    kp = torch.randn((Z, N), generator=g)
    L = bsa.Layout(torch.from_numpy(lay), b)
    _, lse = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), 0.125, True, attn_mask=to_dev(am),
                           key_padding_mask=to_dev(kp), return_lse=True)
    ref = oracle.attention_lse(q, k, lay, b, 0.125, True, am, kp)
    assert _lse_close(lse, ref, 1e-4) <= 1e-4


BWD_CASES = [(b, d, dt, causal) for b in (16, 32, 64, 128) for d in (64, 128) for dt in ("f32", "bf16", "f16")
             for causal in (False, True)]


@pytest.mark.parametrize("b,d,dt,causal", BWD_CASES)
def test_fused_backward(b, d, dt, causal):
    H, nb, Z = 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, 410 + b + d, force_diagonal=True)
    lay[1, 2, :] = 0   # an empty row: zero dq, no contribution to dk, dv
    lay[0, :, 1] = 0   # an empty column: zero dk, dv
    lay[0, 1, 1] = 0
    announce("fused backward", b, d, dt, causal)
    q, k, v, do = _t([(Z, H, nb * b, d)] * 4, 411 + b, dt)
    scale = 1.0 / np.sqrt(d)
    L = bsa.Layout(torch.from_numpy(lay), b)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    o, lse = bsa.attention(L, qd, kd, vd, scale, causal, return_lse=True)
    grads = bsa.attention_backward_fused(L, qd, kd, vd, o, lse, dod, scale, causal)
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, scale, causal)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        assert got.dtype == q.dtype and not torch.isnan(got).any(), name
        assert max_abs(f64(got), ref) <= _grad_tol(dt, ref), name


@pytest.mark.parametrize("b", [16, 64, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("nbr,nbc", [(3, 5), (5, 3)])
def test_fused_backward_nonsquare(b, dt, nbr, nbc):
    """More key blocks than query blocks and the other way round (causal
    needs a square layout and is rejected here)."""
    H, Z, d = 2, 2, 64
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 420 + b + nbr)
    lay[:, :, 0] = 1
    announce("fused backward non-square", b, dt, nbr, nbc)
    g = torch.Generator("cpu").manual_seed(421)
    q, do = (torch.randn((Z, H, nbr * b, d), generator=g).to(DT[dt]) for _ in range(2))
    k, v = (torch.randn((Z, H, nbc * b, d), generator=g).to(DT[dt]) for _ in range(2))
    L = bsa.Layout(torch.from_numpy(lay), b)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    o, lse = bsa.attention(L, qd, kd, vd, 0.125, return_lse=True)
    grads = bsa.attention_backward_fused(L, qd, kd, vd, o, lse, dod, 0.125)
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, 0.125, False)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        assert not torch.isnan(got).any(), name
        assert max_abs(f64(got), ref) <= _grad_tol(dt, ref), name
    with pytest.raises(bsa.BsError):
        bsa.attention_backward_fused(L, qd, kd, vd, o, lse, dod, 0.125, True)


KP_CASES = [(b, 64, dt, causal) for b in (32, 64, 128) for dt in ("bf16", "f16") for causal in (False, True)] + \
    [(128, 128, "bf16", False), (128, 128, "bf16", True), (64, 128, "f16", False)]


@pytest.mark.parametrize("b,d,dt,causal", KP_CASES)
def test_fused_backward_key_padding(b, d, dt, causal):
    """A key-padding mask alone (the 32-row 16-bit kernels read it at 64-
    and 128-blocks): random values, a padded tail of keys, and a batch entry
    whose every key is masked (no gradient at all there)."""
    H, nb, Z = 2, 4, 3
    N = nb * b
    lay = W.small_random_layout(H, nb, nb, 0.5, 460 + b, force_diagonal=True)
    lay[1, 2, :] = 0
    announce("fused backward key padding", b, d, dt, causal)
    q, k, v, do = _t([(Z, H, N, d)] * 4, 461 + b, dt)
    g = torch.Generator("cpu").manual_seed(462)
    kp = torch.randn((Z, N), generator=g) * 0.5
    kp[0, N - N // 3:] = -float("inf")
    kp[1, :] = -float("inf")
    L = bsa.Layout(torch.from_numpy(lay), b)
    qd, kd, vd, dod, kpd = (to_dev(t) for t in (q, k, v, do, kp))
    scale = 1.0 / np.sqrt(d)
    o, lse = bsa.attention(L, qd, kd, vd, scale, causal, key_padding_mask=kpd, return_lse=True)
    grads = bsa.attention_backward_fused(L, qd, kd, vd, o, lse, dod, scale, causal, key_padding_mask=kpd)
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, scale, causal, None, kp)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        assert not torch.isnan(got).any(), name
        assert max_abs(f64(got), ref) <= _grad_tol(dt, ref), name
        assert not got[1].any(), name  # every key of batch entry 1 masked


@pytest.mark.parametrize("b", [32, 64, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("masked", [False, True])
def test_causal_forward_ignores_blocks_above_the_diagonal(b, dt, masked):
    """Causal, the forward walks drop stored blocks wholly above the
    diagonal: output and row log-sum-exp equal, bit for bit, those of the
    same layout without them, and the oracle's."""
    H, nb, Z, d = 2, 5, 2, 64
    N = nb * b
    lay = W.small_random_layout(H, nb, nb, 0.6, 450 + b, force_diagonal=True)
    lay[:, 0, :] = 1
    tri = lay * np.tril(np.ones((nb, nb), np.uint8))[None]
    announce("causal forward above-diagonal blocks", b, dt, masked)
    q, k, v = _t([(Z, H, N, d)] * 3, 451, dt)
    kw, am, kp = {}, None, None
    if masked:
        g = torch.Generator("cpu").manual_seed(452)
        am, kp = torch.randn((N, N), generator=g), torch.randn((Z, N), generator=g) * 0.5
        kw = {"attn_mask": to_dev(am), "key_padding_mask": to_dev(kp)}
    qd, kd, vd = (to_dev(t) for t in (q, k, v))
    L, T = bsa.Layout(torch.from_numpy(lay), b), bsa.Layout(torch.from_numpy(tri), b)
    o, lse = bsa.attention(L, qd, kd, vd, 0.125, True, return_lse=True, **kw)
    o_t, lse_t = bsa.attention(T, qd, kd, vd, 0.125, True, return_lse=True, **kw)
    assert torch.equal(o, o_t) and torch.equal(lse, lse_t)
    ref = oracle.attention_dense(q, k, v, lay, b, 0.125, True, am, kp)
    assert max_abs(f64(o), ref) <= TOL[dt]


@pytest.mark.parametrize("b", [32, 64, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("masked", [False, True])
def test_causal_backward_ignores_blocks_above_the_diagonal(b, dt, masked):
    """Causal, a stored block wholly above the diagonal has P = 0: the
    backward walks drop such blocks, so the gradients equal, bit for bit,
    those of the same layout without them (same forward outputs), and the
    oracle's."""
    H, nb, Z, d = 2, 5, 2, 128
    N = nb * b
    lay = W.small_random_layout(H, nb, nb, 0.6, 440 + b, force_diagonal=True)
    lay[:, 0, :] = 1  # the first block row holds every column (all but one above the diagonal)
    tri = lay * np.tril(np.ones((nb, nb), np.uint8))[None]
    assert (lay != tri).any()
    announce("causal backward above-diagonal blocks", b, dt, masked)
    q, k, v, do = _t([(Z, H, N, d)] * 4, 441, dt)
    kw = {}
    if masked:
        g = torch.Generator("cpu").manual_seed(442)
        kw = {"attn_mask": to_dev(torch.randn((N, N), generator=g)),
              "key_padding_mask": to_dev(torch.randn((Z, N), generator=g) * 0.5)}
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    L, T = bsa.Layout(torch.from_numpy(lay), b), bsa.Layout(torch.from_numpy(tri), b)
    o, lse = bsa.attention(L, qd, kd, vd, 0.125, True, return_lse=True, **kw)
    got = bsa.attention_backward_fused(L, qd, kd, vd, o, lse, dod, 0.125, True, **kw)
    ref_t = bsa.attention_backward_fused(T, qd, kd, vd, o, lse, dod, 0.125, True, **kw)
    am = kw["attn_mask"].cpu() if masked else None
    kp = kw["key_padding_mask"].cpu() if masked else None
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, 0.125, True, am, kp)
    for name, a, c, ref in zip(("dq", "dk", "dv"), got, ref_t, refs):
        assert torch.equal(a, c), name
        assert max_abs(f64(a), ref) <= _grad_tol(dt, ref), name


@pytest.mark.parametrize("b", [16, 64, 128])
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_fused_backward_masked(b, dt, causal):
    H, nb, Z, d = 2, 4, 2, 64
    N = nb * b
    lay = W.small_random_layout(H, nb, nb, 0.5, 430 + b, force_diagonal=True)
    announce("fused backward masked", b, dt, causal)
    q, k, v, do = _t([(Z, H, N, d)] * 4, 431, dt)
    g = torch.Generator("cpu").manual_seed(432)
    am = torch.randn((N, N), generator=g)
    am[torch.rand((N, N), generator=g) < 0.1] = -float("inf")
    am[3, :] = -float("inf")
    kp = torch.randn((Z, N), generator=g) * 0.5
    kp[Z - 1, N - N // 3:] = -float("inf")
    L = bsa.Layout(torch.from_numpy(lay), b)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    amd, kpd = to_dev(am), to_dev(kp)
    o, lse = bsa.attention(L, qd, kd, vd, 0.125, causal, attn_mask=amd, key_padding_mask=kpd, return_lse=True)
    grads = bsa.attention_backward_fused(L, qd, kd, vd, o, lse, dod, 0.125, causal, attn_mask=amd,
                                         key_padding_mask=kpd)
    refs = oracle.attention_backward_dense(q, k, v, do, lay, b, 0.125, causal, am, kp)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        assert not torch.isnan(got).any(), name
        assert max_abs(f64(got), ref) <= _grad_tol(dt, ref), name


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_fused_backward_full_size(idx):
    """causal_b64, bigbird_b64, strided_acsr_b32 (fp32) and
    random_b128_bf16 (the 16-bit kernels, head-grouped order) at full size
    against the dense oracle gradient of every (batch, head) pair. The dense
    route of a random_b128_bf16 head holds about 12 GB of float64 matrices,
    so those heads run four at a time. The gradients are written over NaN,
    and every element must come back finite (nothing left unwritten)."""
    w = W.WORKLOADS[idx]
    lay = W.make_layout(w)
    q, k, v = W.make_qkv(w)
    g = torch.Generator("cpu").manual_seed(440)
    do = torch.randn(q.shape, generator=g).to(q.dtype)
    announce("fused backward full size", w.name)
    L = bsa.Layout(torch.from_numpy(lay), w.block)
    qd, kd, vd, dod = (to_dev(t) for t in (q, k, v, do))
    o, lse = bsa.attention(L, qd, kd, vd, w.scale, w.causal, return_lse=True)
    nan = tuple(torch.full_like(t, float("nan")) for t in (qd, kd, vd))
    dq, dk, dv = bsa.attention_backward_fused(L, qd, kd, vd, o, lse, dod, w.scale, w.causal, out=nan)
    torch.cuda.synchronize()
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(g).all()), ("unwritten gradient", name)
    dt = "f32" if q.dtype == torch.float32 else "bf16"
    pairs = [(z, h) for z in range(w.Z) for h in range(w.H)]
    got = {name: f64(t) for name, t in (("dq", dq), ("dk", dk), ("dv", dv))}

    def check(pair):
        z, h = pair
        sl = (slice(z, z + 1), slice(h, h + 1))
        refs = oracle.attention_backward_dense(q[sl], k[sl], v[sl], do[sl], lay[h:h + 1], w.block, w.scale,
                                               w.causal)
        return [(name, max_abs(got[name][sl], ref), _grad_tol(dt, ref)) for name, ref in zip(("dq", "dk", "dv"), refs)]

    if w.dtype == "f32":
        results = pool_map(check, pairs)
    else:
        from concurrent.futures import ThreadPoolExecutor

        from threadpoolctl import threadpool_limits
        with threadpool_limits(4), ThreadPoolExecutor(4) as ex:
            results = list(ex.map(check, pairs))
    for pair, res in zip(pairs, results):
        for name, err, tol in res:
            assert err <= tol, (name, pair, err)


@pytest.mark.parametrize("b", [64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_fused_backward_16bit_walks_of_zero_and_one_block(b, dt):
    """The 16-bit kernels with nothing to walk (every column and row empty:
    zero gradients in outputs prefilled with NaN) and with one stored block
    per row and column (the dK dV pipeline's shortest walk: two staged
    halves, the dK waves' half one step behind)."""
    d, H, nb, Z = 64, 2, 3, 1
    announce("fused backward 16-bit short walks", b, dt)
    q, k, v, do = (to_dev(t) for t in _t([(Z, H, nb * b, d)] * 4, 460 + b, dt))
    empty = np.zeros((H, nb, nb), np.uint8)
    L = bsa.Layout(torch.from_numpy(empty), b)
    o, lse = bsa.attention(L, q, k, v, 0.125, return_lse=True)
    nan = lambda: torch.full_like(q, float("nan"))
    for g in bsa.attention_backward_fused(L, q, k, v, o, lse, do, 0.125, out=(nan(), nan(), nan())):
        assert torch.all(g == 0)
    perm = np.zeros((H, nb, nb), np.uint8)
    perm[0, np.arange(nb), (np.arange(nb) + 1) % nb] = 1  # one block per row and column
    perm[1, np.arange(nb), np.arange(nb)] = 1
    for causal in (False, True):
        lay = perm if not causal else np.ascontiguousarray(np.broadcast_to(perm[1], perm.shape))
        L = bsa.Layout(torch.from_numpy(lay), b)
        o, lse = bsa.attention(L, q, k, v, 0.125, causal, return_lse=True)
        grads = bsa.attention_backward_fused(L, q, k, v, o, lse, do, 0.125, causal, out=(nan(), nan(), nan()))
        refs = oracle.attention_backward_dense(*(t.cpu() for t in (q, k, v, do)), lay, b, 0.125, causal)
        for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
            assert max_abs(f64(got), ref) <= _grad_tol(dt, ref), (name, causal)


def test_fused_backward_empty_layout_and_empty_batch():
    """No stored block: zero gradients (and -inf lse); Z = 0: nothing to do."""
    b, d, H, nb = 32, 64, 2, 3
    lay = np.zeros((H, nb, nb), np.uint8)
    announce("fused backward empty layout")
    L = bsa.Layout(torch.from_numpy(lay), b)
    q, k, v, do = (to_dev(t) for t in _t([(2, H, nb * b, d)] * 4, 450, "f32"))
    o, lse = bsa.attention(L, q, k, v, 0.125, return_lse=True)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    for g in bsa.attention_backward_fused(L, q, k, v, o, lse, do, 0.125):
        assert torch.all(g == 0)
    e = torch.empty((0, H, nb * b, d), device="cuda")
    o0, lse0 = bsa.attention(L, e, e, e, 0.125, return_lse=True)
    assert o0.shape == e.shape and lse0.shape == (0, H, nb * b)
    for g in bsa.attention_backward_fused(L, e, e, e, o0, lse0, e, 0.125):
        assert g.shape == e.shape
