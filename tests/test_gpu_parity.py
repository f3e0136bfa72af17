"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle.

Small problems are compared element by element; they span several tiles,
every block size, both dtypes, causal and non-causal, ragged contraction
sizes, empty rows/columns and empty layouts. Tolerances: LUT bit-exact;
floating point max-abs 1e-4 (fp32) and 2e-2 (bf16 inputs, fp32 accumulate).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import TOL, announce, f64, max_abs, to_dev

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_matmul_amd")


def _tensors(shape_list, seed, dtype):
    g = torch.Generator("cpu").manual_seed(seed)
    out = []
    for shp in shape_list:
        t = torch.randn(shp, generator=g, dtype=torch.float32)
        if dtype == "bf16":
            t = t.to(torch.bfloat16)
        out.append(t)
    return out


LAYOUT_CASES = [
    ("tiny", lambda: W.make_layout(W.WORKLOADS[0])),
    ("causal", lambda: W.make_layout(W.WORKLOADS[1])),
    ("bigbird", lambda: W.make_layout(W.WORKLOADS[2])),
    ("strided", lambda: W.make_layout(W.WORKLOADS[3])),
    ("random_bf16", lambda: W.make_layout(W.WORKLOADS[4])),
    ("nonsquare_sparse", lambda: W.small_random_layout(3, 7, 13, 0.2, 1)),
    ("all_ones", lambda: np.ones((2, 5, 5), np.uint8)),
    ("all_zeros", lambda: np.zeros((2, 4, 3), np.uint8)),
    ("single", lambda: np.ones((1, 1, 1), np.uint8)),
    ("wide_rows", lambda: W.small_random_layout(2, 3, 300, 0.5, 2)),
    ("tall_cols", lambda: W.small_random_layout(2, 300, 3, 0.5, 3)),
]


@pytest.mark.parametrize("name,make", LAYOUT_CASES, ids=[c[0] for c in LAYOUT_CASES])
def test_lut_bit_exact(name, make):
    lay = make()
    announce("lut", name, lay.shape)
    L = bsa.Layout(torch.from_numpy(lay), 16)
    got = L.export()
    ref = oracle.lut_from_layout(lay)
    assert L.nnz == int(lay.sum())
    for key in ref:
        assert np.array_equal(got[key], ref[key]), key


def test_lut_acsr_bit_exact_strided_workload():
    w = W.workload("strided_acsr_b32")
    announce("lut acsr", w.name)
    L = bsa.Layout.acsr(W.make_acsr(w), w.H, w.nb, w.nb, w.block)
    ref = oracle.lut_from_layout(oracle.acsr_expand(W.make_acsr(w), w.H, w.nb, w.nb))
    got = L.export()
    for key in ref:
        assert np.array_equal(got[key], ref[key]), key
    assert L.nnz == 180736


def test_lut_acsr_clipped_terms():
    terms = [(0, 9, 1, -2, 1, 5), (3, 7, -1, 8, 2, 4), (0, 2, 0, 0, 0, 3), (5, 5, 1, 0, 1, 1)]
    announce("lut acsr clipped")
    L = bsa.Layout.acsr(terms, 2, 9, 6, 32)
    ref = oracle.lut_from_layout(oracle.acsr_expand(terms, 2, 9, 6))
    got = L.export()
    for key in ref:
        assert np.array_equal(got[key], ref[key]), key


def test_lut_rejects_non_binary_values():
    lay = np.zeros((1, 4, 4), np.uint8)
    lay[0, 2, 3] = 3
    announce("lut reject")
    with pytest.raises(bsa.BsError) as e:
        bsa.Layout(torch.from_numpy(lay), 32)
    assert e.value.code == -3


# --------------------------------------------------------------- SDD

# K of 64 and 128 take the LDS-staged row-block kernel, other K the generic one
SDD_CASES = [(b, K, dt) for b in (16, 32, 64, 128)
             for K, dt in ((16, "f32"), (80, "f32"), (64, "f32"), (128, "f32"), (64, "bf16"), (128, "bf16"),
                           (48, "bf16"))]


@pytest.mark.parametrize("b,K,dt", SDD_CASES)
def test_sdd(b, K, dt):
    H, nbr, nbc, Z = 2, 3, 4, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, b + K)
    lay[0, 1, :] = 0  # an empty row
    announce("sdd", b, K, dt)
    a, bb = _tensors([(Z, H, nbr * b, K), (Z, H, nbc * b, K)], 7, dt)
    L = bsa.Layout(torch.from_numpy(lay), b)
    S = bsa.sdd(L, to_dev(a), to_dev(bb))
    ref = oracle.sdd(a, bb, lay, b)
    assert max_abs(f64(S), ref) <= TOL["f32"]


# --------------------------------------------------------------- softmax

@pytest.mark.parametrize("b", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_softmax(b, causal):
    H, nb, Z = 2, 5, 2
    lay = W.small_random_layout(H, nb, nb, 0.45, b)
    lay[1, 2, :] = 0                 # empty row
    lay[0, 0, :] = 0
    lay[0, 0, 3] = 1                 # a row that causal hides completely
    nnz = int(lay.sum())
    announce("softmax", b, causal)
    (S,) = _tensors([(Z, nnz, b, b)], 11, "f32")
    S = S * 3
    L = bsa.Layout(torch.from_numpy(lay), b)
    P = bsa.softmax(L, to_dev(S), 0.7, causal)
    ref = oracle.softmax(S, lay, b, 0.7, causal)
    assert not torch.isnan(P).any()
    assert max_abs(f64(P), ref) <= TOL["f32"]


def test_softmax_in_place_and_long_rows():
    # rows longer than the register cache (re-read path): 300 blocks of 16
    lay = np.ones((1, 2, 300), np.uint8)
    announce("softmax long rows")
    (S,) = _tensors([(1, 600, 16, 16)], 12, "f32")
    L = bsa.Layout(torch.from_numpy(lay), 16)
    Sd = to_dev(S)
    P = bsa.softmax(L, Sd, 0.5, inplace=True)
    assert P.data_ptr() == Sd.data_ptr()
    assert max_abs(f64(P), oracle.softmax(S, lay, 16, 0.5)) <= TOL["f32"]


def _length_class_layout(b, seed):
    """Block rows of every register-cache class of the softmax (up to 8, 16,
    20 and more than 20 cached vectors per lane, i.e. 8*256/b, 16*256/b,
    20*256/b blocks and longer rows), some empty, interleaved over heads and
    rows: a lower-triangular grid of 1.25*20*256/b block rows with rows
    thinned at random and two rows emptied."""
    nb = (20 * 256 // b) * 5 // 4
    rng = np.random.default_rng(seed)
    lay = np.tril(np.ones((2, nb, nb), np.uint8))
    lay &= (rng.random((2, nb, nb)) < rng.uniform(0.3, 1.0, (2, nb, 1))).astype(np.uint8)
    lay[0, nb - 1, :] = 1          # the longest row possible
    lay[0, nb // 2, :] = 0         # empty rows
    lay[1, nb - 3, :] = 0
    return lay


@pytest.mark.parametrize("b", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_softmax_length_classes(b, causal):
    lay = _length_class_layout(b, 40 + b)
    lens = lay.sum(axis=2)
    assert lens.max() * b > 20 * 256 and ((lens > 0) & (lens * b <= 8 * 256)).any()
    assert ((lens * b > 8 * 256) & (lens * b <= 16 * 256)).any()
    assert ((lens * b > 16 * 256) & (lens * b <= 20 * 256)).any()
    nnz = int(lay.sum())
    announce("softmax length classes", b, causal)
    (S,) = _tensors([(2, nnz, b, b)], 41, "f32")
    L = bsa.Layout(torch.from_numpy(lay), b)
    P = bsa.softmax(L, to_dev(S), 0.4, causal)
    ref = oracle.softmax(S, lay, b, 0.4, causal)
    assert max_abs(f64(P), ref) <= TOL["f32"]
    dP = _tensors([(2, nnz, b, b)], 42, "f32")[0]
    dS = bsa.softmax_backward(L, P, to_dev(dP), 0.4)
    assert max_abs(f64(dS), oracle.softmax_backward(f64(P), dP, lay, b, 0.4)) <= TOL["f32"]


# --------------------------------------------------------------- DSD / DDS

# Nd of 64 and 128 take the LDS-staged row-block kernel, other Nd the generic one
DSD_CASES = [(b, n, dt) for b in (16, 32, 64, 128)
             for n, dt in ((64, "f32"), (128, "f32"), (48, "f32"), (64, "bf16"), (128, "bf16"), (16, "bf16"))]


@pytest.mark.parametrize("b,Nd,dt", DSD_CASES)
def test_dsd(b, Nd, dt):
    H, nbr, nbc, Z = 2, 4, 3, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, b + Nd)
    lay[1, 3, :] = 0
    nnz = int(lay.sum())
    announce("dsd", b, Nd, dt)
    (Bm,) = _tensors([(Z, H, nbc * b, Nd)], 13, dt)
    g = torch.Generator("cpu").manual_seed(14)
    P = torch.rand((Z, nnz, b, b), generator=g) / b  # probability-like
    L = bsa.Layout(torch.from_numpy(lay), b)
    C = bsa.dsd(L, to_dev(P), to_dev(Bm))
    assert C.dtype == Bm.dtype
    ref = oracle.dsd(P, Bm, lay, b)
    assert max_abs(f64(C), ref) <= TOL[dt]


# M beyond 64 spans several 64-row chunks of the DDS grid (112, 80: a partial last chunk)
DDS_CASES = [(b, m, dt) for b in (16, 32, 64, 128)
             for m, dt in ((64, "f32"), (16, "f32"), (112, "f32"), (32, "bf16"), (48, "bf16"), (80, "bf16"))]


@pytest.mark.parametrize("b,M,dt", DDS_CASES)
def test_dds(b, M, dt):
    H, nbr, nbc, Z = 2, 3, 5, 2
    lay = W.small_random_layout(H, nbr, nbc, 0.5, b + M + 1)
    lay[0, :, 2] = 0  # an empty column
    nnz = int(lay.sum())
    announce("dds", b, M, dt)
    (A,) = _tensors([(Z, H, M, nbr * b)], 15, dt)
    g = torch.Generator("cpu").manual_seed(16)
    S = torch.rand((Z, nnz, b, b), generator=g) / b
    L = bsa.Layout(torch.from_numpy(lay), b)
    C = bsa.dds(L, to_dev(A), to_dev(S))
    ref = oracle.dds(A, S, lay, b)
    assert max_abs(f64(C), ref) <= TOL[dt]


@pytest.mark.parametrize("b", [16, 32, 128])
def test_dds_random_values_relative(b):
    """Long columns (several 64- or 128-row slabs, which span several blocks
    for small b) with N(0,1) block values: fp32 rounding grows with the
    column length, so the bound is relative to the largest output (1e-4 of
    max |C|)."""
    M = 64
    lay = W.small_random_layout(2, 40, 6, 0.7, 17)
    nnz = int(lay.sum())
    announce("dds random relative", b)
    A, S = _tensors([(1, 2, M, 40 * b), (1, nnz, b, b)], 18, "f32")
    L = bsa.Layout(torch.from_numpy(lay), b)
    C = bsa.dds(L, to_dev(A), to_dev(S))
    ref = oracle.dds(A, S, lay, b)
    assert max_abs(f64(C), ref) <= 1e-4 * np.abs(ref).max()


@pytest.mark.parametrize("b", [16, 64])
def test_dds_long_columns_bf16(b):
    """bf16 over long columns whose length in 16-row tiles is odd (b = 16:
    the last 32-deep product is half padding)."""
    M = 48
    lay = W.small_random_layout(2, 41, 5, 0.7, 19)
    lay[:, :, 0] = 1  # 41 blocks: an odd tile count for b = 16
    nnz = int(lay.sum())
    announce("dds long columns bf16", b)
    (A,) = _tensors([(2, 2, M, 41 * b)], 20, "bf16")
    g = torch.Generator("cpu").manual_seed(21)
    S = torch.rand((2, nnz, b, b), generator=g) / b
    L = bsa.Layout(torch.from_numpy(lay), b)
    C = bsa.dds(L, to_dev(A), to_dev(S))
    ref = oracle.dds(A, S, lay, b)
    assert max_abs(f64(C), ref) <= TOL["bf16"]


# --------------------------------------------------------------- attention

ATTN_CASES = [(b, d, dt, causal) for b in (16, 32, 64, 128) for d in (64, 128) for dt in ("f32", "bf16")
              for causal in (False, True)]


@pytest.mark.parametrize("b,d,dt,causal", ATTN_CASES)
def test_attention_small(b, d, dt, causal):
    H, nb, Z = 2, 4, 2
    lay = W.small_random_layout(H, nb, nb, 0.5, b + d, force_diagonal=True)
    lay[1, 2, :] = 0   # empty row -> zeros
    lay[0, 0, :] = 0
    lay[0, 0, 2] = 1   # causal hides this row completely -> zeros
    announce("attention", b, d, dt, causal)
    q, k, v = _tensors([(Z, H, nb * b, d)] * 3, b * d, dt)
    scale = 1.0 / np.sqrt(d)
    L = bsa.Layout(torch.from_numpy(lay), b)
    O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), scale, causal)
    assert O.dtype == q.dtype
    ref = oracle.attention_dense(q, k, v, lay, b, scale, causal)
    assert not torch.isnan(O).any()
    assert max_abs(f64(O), ref) <= TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_unfused_chain_matches_fused_and_oracle(dt):
    b, d, H, nb, Z = 32, 64, 3, 6, 2
    lay = W.small_random_layout(H, nb, nb, 0.4, 21, force_diagonal=True)
    announce("unfused chain", dt)
    q, k, v = _tensors([(Z, H, nb * b, d)] * 3, 22, dt)
    L = bsa.Layout(torch.from_numpy(lay), b)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    S = bsa.sdd(L, qd, kd)
    P = bsa.softmax(L, S, 0.125, causal=True)
    O1 = bsa.dsd(L, P, vd)
    O2 = bsa.attention(L, qd, kd, vd, 0.125, causal=True)
    ref = oracle.attention_dense(q, k, v, lay, b, 0.125, True)
    assert max_abs(f64(O1), ref) <= TOL[dt]
    assert max_abs(f64(O2), ref) <= TOL[dt]


def test_empty_layout_outputs_zero():
    lay = np.zeros((2, 3, 3), np.uint8)
    announce("empty layout")
    L = bsa.Layout(torch.from_numpy(lay), 64)
    assert L.nnz == 0
    q = torch.randn(1, 2, 192, 64, device="cuda")
    O = bsa.attention(L, q, q, q)
    assert torch.count_nonzero(O) == 0
    S = torch.empty((1, 0, 64, 64), device="cuda")
    C = bsa.dsd(L, S, q)
    assert torch.count_nonzero(C) == 0
    a = torch.randn(1, 2, 32, 192, device="cuda")
    C2 = bsa.dds(L, a, S)
    assert torch.count_nonzero(C2) == 0


def test_deterministic_repeat():
    w = W.WORKLOADS[0]
    lay = W.make_layout(w)
    announce("determinism")
    q, k, v = (to_dev(t) for t in W.make_qkv(w))
    L = bsa.Layout(torch.from_numpy(lay), w.block)
    O1 = bsa.attention(L, q, k, v, w.scale)
    O2 = bsa.attention(L, q, k, v, w.scale)
    assert torch.equal(O1, O2)
    S1, S2 = bsa.sdd(L, q, k), bsa.sdd(L, q, k)
    assert torch.equal(S1, S2)


def test_errors_from_python_binding():
    lay = np.ones((1, 2, 2), np.uint8)
    L = bsa.Layout(torch.from_numpy(lay), 16)
    q = torch.randn(1, 1, 32, 64, device="cuda")
    with pytest.raises(ValueError):
        bsa.attention(L, q, q, q[:, :, :16])
    with pytest.raises(bsa.BsError) as e:
        bsa.attention(L, q[..., :48].contiguous(), q[..., :48].contiguous(), q[..., :48].contiguous())
    assert e.value.code == -2
    Lr = bsa.Layout(torch.from_numpy(np.ones((1, 2, 3), np.uint8)), 16)
    k = torch.randn(1, 1, 48, 64, device="cuda")
    with pytest.raises(bsa.BsError) as e:
        bsa.attention(Lr, q, k, k, causal=True)
    assert e.value.code == -1


@pytest.mark.parametrize("b", [16, 32, 64])
@pytest.mark.parametrize("Z", [1, 128, 256])
def test_attention_batch_sweep_all_key_group_schedules(b, Z):
    """The fused kernel splits a row's blocks over 1, 2 or 4 key groups of
    waves depending on how long the longest row is against the work per
    CU; a batch sweep on one layout exercises every choice. Checked on
    sampled block rows against the oracle."""
    H, nb, d = 2, 4, 64
    lay = W.small_random_layout(H, nb, nb, 0.5, 50 + b, force_diagonal=True)
    announce("attention batch sweep", b, Z)
    q, k, v = _tensors([(Z, H, nb * b, d)] * 3, 51, "f32")
    L = bsa.Layout(torch.from_numpy(lay), b)
    for causal in (False, True):
        O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), 0.125, causal)
        rows = [(0, 0, 0), (Z - 1, 1, nb - 1), (Z // 2, 0, 2), (Z // 3, 1, 1)]
        ref = oracle.attention_rows(q, k, v, lay, b, 0.125, causal, rows)
        for n, (z, h, r) in enumerate(rows):
            assert max_abs(f64(O[z, h, r * b:(r + 1) * b]), ref[n]) <= TOL["f32"], (z, h, r, causal)


@pytest.mark.parametrize("b", [16, 32, 64])
@pytest.mark.parametrize("Z", [1, 128, 256])
def test_ops_batch_sweep_all_key_group_schedules(b, Z):
    """SDD, DSD (on the row-block kernel) and DDS split a row's or column's
    blocks over 1, 2 or 4 key groups depending on its length against the
    work per CU; a batch sweep on one layout exercises every choice. Checked
    on sampled batch entries against the oracle."""
    H, nb, d = 2, 4, 64
    lay = W.small_random_layout(H, nb, nb, 0.5, 60 + b, force_diagonal=True)
    nnz = int(lay.sum())
    announce("ops batch sweep", b, Z)
    a, bb, dense = _tensors([(Z, H, nb * b, d), (Z, H, nb * b, d), (Z, H, d, nb * b)], 61, "f32")
    g = torch.Generator("cpu").manual_seed(62)
    P = torch.rand((Z, nnz, b, b), generator=g) / b
    L = bsa.Layout(torch.from_numpy(lay), b)
    S = bsa.sdd(L, to_dev(a), to_dev(bb))
    C = bsa.dsd(L, to_dev(P), to_dev(bb))
    D = bsa.dds(L, to_dev(dense), to_dev(P))
    for z in sorted({0, Z // 3, Z // 2, Z - 1}):
        sl = slice(z, z + 1)
        assert max_abs(f64(S[sl]), oracle.sdd(a[sl], bb[sl], lay, b)) <= TOL["f32"], ("sdd", z)
        assert max_abs(f64(C[sl]), oracle.dsd(P[sl], bb[sl], lay, b)) <= TOL["f32"], ("dsd", z)
        assert max_abs(f64(D[sl]), oracle.dds(dense[sl], P[sl], lay, b)) <= TOL["f32"], ("dds", z)


BF16_SWEEP = [(32, 1), (32, 80), (32, 256), (64, 1), (64, 80), (64, 256), (128, 1), (128, 40), (128, 256)]


@pytest.mark.parametrize("b,Z", BF16_SWEEP)
@pytest.mark.parametrize("d", [64, 128])
def test_attention_bf16_batch_sweep_all_key_group_schedules(b, Z, d):
    """bf16 attention with blocks of 32 to 128 runs on the kernel with 32
    query rows per wave; its key-group count (1, 2 or 4, as the LDS allows)
    follows the batch size the same way. Sampled block rows against the
    oracle, causal and not."""
    H, nb = 2, 4
    lay = W.small_random_layout(H, nb, nb, 0.5, 50 + b, force_diagonal=True)
    announce("attention bf16 batch sweep", b, Z, d)
    q, k, v = _tensors([(Z, H, nb * b, d)] * 3, 52, "bf16")
    L = bsa.Layout(torch.from_numpy(lay), b)
    scale = 1.0 / np.sqrt(d)
    for causal in (False, True):
        O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), scale, causal)
        rows = [(0, 0, 0), (Z - 1, 1, nb - 1), (Z // 2, 0, 2), (Z // 3, 1, 1)]
        ref = oracle.attention_rows(q, k, v, lay, b, scale, causal, rows)
        for n, (z, h, r) in enumerate(rows):
            assert max_abs(f64(O[z, h, r * b:(r + 1) * b]), ref[n]) <= TOL["bf16"], (z, h, r, causal)


@pytest.mark.parametrize("b", [32, 64, 128])
def test_attention_bf16_head_grouped_order(b):
    """When no row is long against a workgroup's share of the job, the bf16
    kernel walks the rows grouped by (batch, head), one contiguous range per
    XCD; a dense layout with a large batch takes that order. Sampled block
    rows across batch entries and heads against the oracle."""
    H, nb, d, Z = 2, 4, 128, 256
    lay = np.ones((H, nb, nb), np.uint8)
    announce("attention bf16 head-grouped order", b)
    q, k, v = _tensors([(Z, H, nb * b, d)] * 3, 53, "bf16")
    L = bsa.Layout(torch.from_numpy(lay), b)
    scale = 1.0 / np.sqrt(d)
    for causal in (False, True):
        O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), scale, causal)
        rows = [(0, 0, 0), (Z - 1, 1, nb - 1), (Z // 2, 0, 2), (Z // 3, 1, 1), (7, 1, 3), (130, 0, 1)]
        ref = oracle.attention_rows(q, k, v, lay, b, scale, causal, rows)
        for n, (z, h, r) in enumerate(rows):
            assert max_abs(f64(O[z, h, r * b:(r + 1) * b]), ref[n]) <= TOL["bf16"], (z, h, r, causal)
