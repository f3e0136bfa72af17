"""Pins for the oracle's SDD, softmax, DSD, DDS and attention.

What the pages fix (Triton issue 117, "question on blocksparse"): SDD output
is block-sparse and feeds softmax and DSD; the block-sparse softmax is the
same as full-attention softmax; a block-triangular layout plus a dense mask on
the diagonal blocks is causal attention. The streaming recurrence of the
Triton tutorial (Puzzle 8, online softmax; Puzzle 9, simple FlashAttention)
equals the two-pass softmax. Every pin below is either a special case that
reduces to a library routine (numpy matmul, torch softmax / SDPA), a closed
form, an invariant, or brute force with explicit loops.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _ones(H, nbr, nbc):
    return np.ones((H, nbr, nbc), dtype=np.uint8)


# ------------------------------------------------------------------ SDD

@pytest.mark.parametrize("b", [16, 32])
def test_sdd_all_ones_is_dense_product(b):
    Z, H, nb, K = 2, 2, 3, 24
    A, B = _rand((Z, H, nb * b, K), 1), _rand((Z, H, nb * b, K), 2)
    S = oracle.sdd(A, B, _ones(H, nb, nb), b)
    dense = A @ np.swapaxes(B, 2, 3)            # numpy matmul, [Z, H, N, N]
    k = 0
    for h in range(H):
        for r in range(nb):
            for c in range(nb):
                assert np.allclose(S[:, k], dense[:, h, r * b:(r + 1) * b, c * b:(c + 1) * b], atol=1e-12)
                k += 1


def test_sdd_brute_force_loops():
    b, Z, H, nb, K = 16, 1, 2, 2, 5
    lay = W.small_random_layout(H, nb, nb, 0.5, 7, force_diagonal=True)
    A, B = _rand((Z, H, nb * b, K), 3), _rand((Z, H, nb * b, K), 4)
    S = oracle.sdd(A, B, lay, b)
    k = 0
    for h in range(H):
        for r in range(nb):
            for c in range(nb):
                if not lay[h, r, c]:
                    continue
                for i in range(b):
                    for j in range(b):
                        acc = 0.0
                        for t in range(K):
                            acc += A[0, h, r * b + i, t] * B[0, h, c * b + j, t]
                        assert abs(S[0, k, i, j] - acc) < 1e-12
                k += 1


# ------------------------------------------------------------------ softmax

def test_softmax_all_ones_equals_torch_softmax():
    b, Z, H, nb, scale = 16, 2, 3, 3, 0.37
    S_dense = _rand((Z, H, nb * b, nb * b), 5)
    lay = _ones(H, nb, nb)
    # block-sparse form of the dense matrix, in block-id order
    S = np.stack([np.stack([S_dense[z, h, r * b:(r + 1) * b, c * b:(c + 1) * b]
                            for h in range(H) for r in range(nb) for c in range(nb)]) for z in range(Z)])
    P = oracle.softmax(S, lay, b, scale)
    ref = torch.softmax(torch.from_numpy(scale * S_dense), dim=-1).numpy()
    k = 0
    for h in range(H):
        for r in range(nb):
            for c in range(nb):
                assert np.allclose(P[:, k], ref[:, h, r * b:(r + 1) * b, c * b:(c + 1) * b], atol=1e-14)
                k += 1


def test_softmax_causal_lower_triangular_equals_masked_torch_softmax():
    b, nb, scale = 16, 4, 0.5
    S_dense = _rand((1, 1, nb * b, nb * b), 6)
    lay = np.tril(np.ones((nb, nb), dtype=np.uint8))[None]
    blocks = [(r, c) for r in range(nb) for c in range(nb) if c <= r]
    S = np.stack([S_dense[0, 0, r * b:(r + 1) * b, c * b:(c + 1) * b] for r, c in blocks])[None]
    P = oracle.softmax(S, lay, b, scale, causal=True)
    x = torch.from_numpy(scale * S_dense[0, 0])
    x = x.masked_fill(torch.triu(torch.ones_like(x, dtype=torch.bool), 1), float("-inf"))
    ref = torch.softmax(x, dim=-1).numpy()
    for k, (r, c) in enumerate(blocks):
        assert np.allclose(P[0, k], ref[r * b:(r + 1) * b, c * b:(c + 1) * b], atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one_and_shift_invariance(causal):
    b, H, nb, scale = 16, 3, 5, 0.25
    lay = W.small_random_layout(H, nb, nb, 0.4, 9, force_diagonal=True)
    nnz = int(lay.sum())
    S = _rand((2, nnz, b, b), 10)
    P = oracle.softmax(S, lay, b, scale, causal)
    lut = oracle.lut_from_layout(lay)
    rp = lut["row_ptr"]
    for hr in range(H * nb):
        ks = range(rp[hr], rp[hr + 1])
        rowsum = sum(P[:, k].sum(axis=2) for k in ks)
        assert np.allclose(rowsum, 1.0, atol=1e-13)
    # adding a per-row constant to every stored entry of a row changes nothing
    shift = _rand((2, H * nb, b), 11) * 7
    S2 = S.copy()
    for hr in range(H * nb):
        for k in range(rp[hr], rp[hr + 1]):
            S2[:, k] += shift[:, hr, :, None] / scale
    assert np.allclose(oracle.softmax(S2, lay, b, scale, causal), P, atol=1e-12)
    assert np.all(P >= 0)


def test_softmax_empty_and_fully_masked_rows_are_zero():
    b = 16
    lay = np.zeros((1, 3, 3), dtype=np.uint8)
    lay[0, 0, 2] = 1      # above the diagonal: fully hidden under causal
    lay[0, 2, 0] = 1      # visible
    S = _rand((1, 2, b, b), 12)
    P = oracle.softmax(S, lay, b, 1.0, causal=True)
    assert np.all(P[0, 0] == 0)
    assert np.allclose(P[0, 1].sum(axis=1), 1.0)
    assert not np.any(np.isnan(P))


def test_softmax_two_pass_equals_streaming_recurrence():
    """The streaming form of the Triton tutorial (Puzzle 8): visit a row in
    tiles, keep a running max m and a running sum l rescaled by exp(m_old -
    m_new); the final exp(x - m)/l equals the oracle's two-pass softmax."""
    b, nb, scale = 16, 4, 0.8
    lay = np.ones((1, 1, nb), dtype=np.uint8)
    S = _rand((1, nb, b, b), 13)
    P = oracle.softmax(S, lay, b, scale)
    x = scale * np.concatenate([S[0, k] for k in range(nb)], axis=1)
    m = np.full(b, -np.inf)
    l = np.zeros(b)
    for t in range(nb):
        tile = x[:, t * b:(t + 1) * b]
        m_new = np.maximum(m, tile.max(axis=1))
        l = l * np.exp(m - m_new) + np.exp(tile - m_new[:, None]).sum(axis=1)
        m = m_new
    stream = np.exp(x - m[:, None]) / l[:, None]
    assert np.allclose(np.concatenate([P[0, k] for k in range(nb)], axis=1), stream, atol=1e-14)


# ------------------------------------------------------------------ DSD

def test_dsd_all_ones_is_dense_product():
    b, Z, H, nb, Nd = 16, 2, 2, 3, 20
    lay = _ones(H, nb, nb)
    P_dense = _rand((Z, H, nb * b, nb * b), 14)
    P = np.stack([np.stack([P_dense[z, h, r * b:(r + 1) * b, c * b:(c + 1) * b]
                            for h in range(H) for r in range(nb) for c in range(nb)]) for z in range(Z)])
    B = _rand((Z, H, nb * b, Nd), 15)
    assert np.allclose(oracle.dsd(P, B, lay, b), P_dense @ B, atol=1e-12)


def test_dsd_identity_blocks_copy_and_empty_rows_zero():
    b, nb, Nd = 16, 4, 8
    lay = np.zeros((1, nb, nb), dtype=np.uint8)
    lay[0, 0, 3] = 1
    lay[0, 2, 1] = 1           # rows 1 and 3 are empty
    P = np.stack([np.eye(b), np.eye(b)])[None]
    B = _rand((1, 1, nb * b, Nd), 16)
    C = oracle.dsd(P, B, lay, b)
    assert np.array_equal(C[0, 0, 0:b], B[0, 0, 3 * b:4 * b])
    assert np.array_equal(C[0, 0, 2 * b:3 * b], B[0, 0, b:2 * b])
    assert np.all(C[0, 0, b:2 * b] == 0) and np.all(C[0, 0, 3 * b:] == 0)


# ------------------------------------------------------------------ DDS

def test_dds_all_ones_is_dense_product():
    b, Z, H, nb, M = 16, 2, 2, 3, 12
    lay = _ones(H, nb, nb)
    S_dense = _rand((Z, H, nb * b, nb * b), 17)
    S = np.stack([np.stack([S_dense[z, h, r * b:(r + 1) * b, c * b:(c + 1) * b]
                            for h in range(H) for r in range(nb) for c in range(nb)]) for z in range(Z)])
    A = _rand((Z, H, M, nb * b), 18)
    assert np.allclose(oracle.dds(A, S, lay, b), A @ S_dense, atol=1e-12)


def test_dds_is_transposed_dsd():
    """(A S)^T = S^T A^T: DDS on layout L equals DSD on the transposed layout
    with every block transposed; the transposed layout enumerates blocks in
    the CSC order of L, so its k-th block is S[blk_id[k]]^T."""
    b, Z, H, nbr, nbc, M = 16, 2, 3, 4, 5, 10
    lay = W.small_random_layout(H, nbr, nbc, 0.35, 19)
    nnz = int(lay.sum())
    S = _rand((Z, nnz, b, b), 20)
    A = _rand((Z, H, M, nbr * b), 21)
    C = oracle.dds(A, S, lay, b)
    lut = oracle.lut_from_layout(lay)
    S_t = np.swapaxes(S[:, lut["blk_id"]], 2, 3)
    lay_t = np.ascontiguousarray(np.transpose(lay, (0, 2, 1)))
    C_t = oracle.dsd(S_t, np.swapaxes(A, 2, 3), lay_t, b)
    assert np.allclose(C, np.swapaxes(C_t, 2, 3), atol=1e-12)


# ------------------------------------------------------------------ attention

def _sdpa(q, k, v, scale, causal=False, mask=None):
    t = [torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(
        *t, attn_mask=None if mask is None else torch.from_numpy(mask),
        is_causal=causal, scale=scale).numpy()


def test_attention_all_ones_equals_sdpa():
    b, Z, H, nb, d = 16, 2, 2, 4, 32
    q, k, v = (_rand((Z, H, nb * b, d), s) for s in (22, 23, 24))
    scale = 1 / math.sqrt(d)
    lay = _ones(H, nb, nb)
    ref = _sdpa(q, k, v, scale)
    assert np.allclose(oracle.attention_dense(q, k, v, lay, b, scale), ref, atol=1e-12)
    assert np.allclose(oracle.attention_blocks(q, k, v, lay, b, scale), ref, atol=1e-12)


def test_attention_lower_triangular_causal_equals_causal_sdpa():
    b, Z, H, nb, d = 16, 1, 2, 5, 16
    q, k, v = (_rand((Z, H, nb * b, d), s) for s in (25, 26, 27))
    scale = 0.3
    lay = W.lower_triangular_layout(H, nb)
    ref = _sdpa(q, k, v, scale, causal=True)
    assert np.allclose(oracle.attention_dense(q, k, v, lay, b, scale, True), ref, atol=1e-12)
    assert np.allclose(oracle.attention_blocks(q, k, v, lay, b, scale, True), ref, atol=1e-12)


def test_attention_block_diagonal_is_per_block_attention():
    b, Z, H, nb, d = 32, 2, 2, 3, 16
    q, k, v = (_rand((Z, H, nb * b, d), s) for s in (28, 29, 30))
    scale = 0.25
    lay = np.broadcast_to(np.eye(nb, dtype=np.uint8), (H, nb, nb)).copy()
    O = oracle.attention_blocks(q, k, v, lay, b, scale)
    for r in range(nb):
        sl = slice(r * b, (r + 1) * b)
        assert np.allclose(O[:, :, sl], _sdpa(q[:, :, sl], k[:, :, sl], v[:, :, sl], scale), atol=1e-12)


def test_attention_brute_force_loops():
    b, nb, d = 16, 2, 3
    lay = np.array([[[1, 0], [1, 1]]], dtype=np.uint8)
    q, k, v = (_rand((1, 1, nb * b, d), s) for s in (31, 32, 33))
    scale = 0.9
    for causal in (False, True):
        O = oracle.attention_blocks(q, k, v, lay, b, scale, causal)
        for i in range(nb * b):
            vis = [j for j in range(nb * b) if lay[0, i // b, j // b] and (not causal or j <= i)]
            sc = [scale * sum(q[0, 0, i, t] * k[0, 0, j, t] for t in range(d)) for j in vis]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            tot = sum(w)
            for n in range(d):
                ref = sum(wj * v[0, 0, j, n] for wj, j in zip(w, vis)) / tot
                assert abs(O[0, 0, i, n] - ref) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_attention_closed_form_zero_queries_average_values(causal):
    """Q = 0 makes every visible score equal, so each output row is the mean
    of the visible value rows."""
    b, H, nb, d = 16, 2, 4, 8
    lay = W.small_random_layout(H, nb, nb, 0.5, 34, force_diagonal=True)
    q = np.zeros((1, H, nb * b, d))
    k, v = _rand((1, H, nb * b, d), 35), _rand((1, H, nb * b, d), 36)
    O = oracle.attention_blocks(q, k, v, lay, b, 1.0, causal)
    mask = oracle.element_mask(lay, b, causal)
    for h in range(H):
        ref = (mask[h] @ v[0, h]) / mask[h].sum(axis=1, keepdims=True)
        assert np.allclose(O[0, h], ref, atol=1e-13)


def test_attention_routes_agree_on_workload_shapes():
    """Route (i) dense-masked and route (ii) per-block agree to 1e-12 on the
    tiny workload and on a cut-down causal/bigbird style problem; the sampled
    row helpers agree with both."""
    w = W.workload("tiny_b16")
    lay = W.make_layout(w)
    q, k, v = W.make_qkv(w)
    Od = oracle.attention_dense(q, k, v, lay, w.block, w.scale)
    Ob = oracle.attention_blocks(q, k, v, lay, w.block, w.scale)
    assert np.max(np.abs(Od - Ob)) < 1e-12
    rows = [(0, 0, r) for r in (0, 5, 15)]
    Or = oracle.attention_rows(q, k, v, lay, w.block, w.scale, False, rows)
    for n, (z, h, r) in enumerate(rows):
        sl = slice(r * w.block, (r + 1) * w.block)
        assert np.max(np.abs(Or[n] - Od[z, h, sl])) < 1e-12
        br = oracle.attention_blockrow(q, k, v, lay, w.block, w.scale, False, z, h, r)
        assert np.max(np.abs(br - Od[z, h, sl])) < 1e-12
    # causal, several heads and a batch
    lay = W.lower_triangular_layout(3, 4)
    q, k, v = (_rand((2, 3, 64, 16), s) for s in (37, 38, 39))
    Od = oracle.attention_dense(q, k, v, lay, 16, 0.25, True)
    Ob = oracle.attention_blocks(q, k, v, lay, 16, 0.25, True)
    assert np.max(np.abs(Od - Ob)) < 1e-12
    Or = oracle.attention_rows(q, k, v, lay, 16, 0.25, True, [(1, 2, 3), (0, 1, 0)])
    assert np.max(np.abs(Or[0] - Od[1, 2, 48:64])) < 1e-12
    assert np.max(np.abs(Or[1] - Od[0, 1, 0:16])) < 1e-12


def test_attention_empty_row_gives_zero_not_nan():
    b = 16
    lay = np.zeros((1, 2, 2), dtype=np.uint8)
    lay[0, 1, 0] = 1
    q, k, v = (_rand((1, 1, 32, 8), s) for s in (40, 41, 42))
    for fn in (oracle.attention_dense, oracle.attention_blocks):
        O = fn(q, k, v, lay, b, 1.0)
        assert np.all(O[0, 0, :16] == 0) and not np.any(np.isnan(O))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_rows_and_blockrow_match_dense_on_per_head_layouts(causal):
    """Every block row of a per-head random layout: the sampled-row routes
    equal the full dense-masked route."""
    b, Z, H, nb, d = 16, 2, 3, 4, 8
    lay = W.small_random_layout(H, nb, nb, 0.45, 43, force_diagonal=True)
    q, k, v = (_rand((Z, H, nb * b, d), s) for s in (44, 45, 46))
    Od = oracle.attention_dense(q, k, v, lay, b, 0.5, causal)
    rows = [(z, h, r) for z in range(Z) for h in range(H) for r in range(nb)]
    Or = oracle.attention_rows(q, k, v, lay, b, 0.5, causal, rows)
    for n, (z, h, r) in enumerate(rows):
        sl = slice(r * b, (r + 1) * b)
        assert np.max(np.abs(Or[n] - Od[z, h, sl])) < 1e-12
        br = oracle.attention_blockrow(q, k, v, lay, b, 0.5, causal, z, h, r)
        assert np.max(np.abs(br - Od[z, h, sl])) < 1e-12
