"""Pins for the oracle's backward: softmax_backward, dsd_t and the attention
gradient.

The gradient is the exact derivative of the forward, so the pins are: central
finite differences of the oracle's own forward in float64 (an independent
route: it never uses the backward formulas), torch's autograd through the
math path of scaled_dot_product_attention in float64 on the CPU (a library
routine computing the same gradient), the transposed-layout identity for
dsd_t (DSD on the transposed block matrix), a dense closed form, and the
agreement of the two oracle routes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _layout_with_empty_row(H, nb, seed):
    lay = W.small_random_layout(H, nb, nb, 0.5, seed, force_diagonal=True)
    lay[0, 1, :] = 0  # an empty block row: its output and gradients are zero
    return lay


def _numeric_grad(f, x, eps=1e-6):
    """Central differences of the scalar f at every element of x (float64)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


# ------------------------------------------------------------ finite differences

@pytest.mark.parametrize("causal", [False, True])
def test_attention_gradient_matches_finite_differences(causal):
    Z, H, nb, b, d = 1, 2, 2, 16, 4
    lay = _layout_with_empty_row(H, nb, 3)
    Q, K, V = _rand((Z, H, nb * b, d), 4), _rand((Z, H, nb * b, d), 5), _rand((Z, H, nb * b, d), 6)
    G = _rand((Z, H, nb * b, d), 7)  # dL/dO of the loss L = sum(O * G)
    scale = 0.4

    def loss():
        return float((oracle.attention_dense(Q, K, V, lay, b, scale, causal) * G).sum())

    dQ, dK, dV = oracle.attention_backward_dense(Q, K, V, G, lay, b, scale, causal)
    for name, x, g in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        num = _numeric_grad(loss, x)
        assert np.abs(num - g).max() <= 1e-6 * max(1.0, np.abs(num).max()), name


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_backward_matches_finite_differences(causal):
    Z, H, nb, b = 1, 2, 2, 16
    lay = _layout_with_empty_row(H, nb, 8)
    nnz = int(lay.sum())
    S = _rand((Z, nnz, b, b), 9) * 2
    G = _rand((Z, nnz, b, b), 10)
    scale = 0.7

    def loss():
        return float((oracle.softmax(S, lay, b, scale, causal) * G).sum())

    P = oracle.softmax(S, lay, b, scale, causal)
    dS = oracle.softmax_backward(P, G, lay, b, scale)
    num = _numeric_grad(loss, S)
    assert np.abs(num - dS).max() <= 1e-6 * max(1.0, np.abs(num).max())


# ------------------------------------------------------------ library routine

@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_gradient_is_sdpa_autograd(causal):
    """A dense layout (with is_causal for the causal mask) is plain attention:
    torch autograd through SDPA's math path in float64 gives the gradient."""
    Z, H, nb, b, d = 2, 2, 3, 16, 8
    lay = np.ones((H, nb, nb), np.uint8)
    Q, K, V, G = (_rand((Z, H, nb * b, d), s) for s in (11, 12, 13, 14))
    scale = 1 / np.sqrt(d)
    dQ, dK, dV = oracle.attention_backward_dense(Q, K, V, G, lay, b, scale, causal)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    from torch.nn.attention import SDPBackend, sdpa_kernel
    with sdpa_kernel(SDPBackend.MATH):
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
    o.backward(torch.tensor(G))
    for name, ours, ref in (("Q", dQ, q.grad), ("K", dK, k.grad), ("V", dV, v.grad)):
        assert np.abs(ours - ref.numpy()).max() < 1e-10, name


# ------------------------------------------------------------ dsd_t

def _transposed(lay, S):
    """The transposed block matrix: layout L^T[h, c, r] = L[h, r, c] and its
    blocks S^T, renumbered in L^T's (head, row, col) order, which is L's CSC
    order (blk_id maps a CSC position to the CSR block id)."""
    lut = oracle.lut_from_layout(lay)
    ST = np.stack([np.swapaxes(S[:, int(k)], 1, 2) for k in lut["blk_id"]], axis=1)
    return np.ascontiguousarray(np.swapaxes(lay, 1, 2)), ST


@pytest.mark.parametrize("b", [16, 32])
def test_dsd_t_is_dsd_of_the_transposed_block_matrix(b):
    H, nbr, nbc, Z, Nd = 2, 3, 4, 2, 8
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 15 + b)
    lay[1, :, 2] = 0  # an empty block column: zero rows of the output
    nnz = int(lay.sum())
    S = _rand((Z, nnz, b, b), 16)
    B = _rand((Z, H, nbr * b, Nd), 17)
    layT, ST = _transposed(lay, S)
    C = oracle.dsd_t(S, B, lay, b)
    assert np.abs(C - oracle.dsd(ST, B, layT, b)).max() < 1e-12
    assert np.all(C[:, 1, 2 * b:3 * b] == 0)


def test_dsd_t_all_ones_is_dense_transposed_product():
    H, nb, b, Z, Nd = 1, 3, 16, 1, 5
    lay = np.ones((H, nb, nb), np.uint8)
    S = _rand((Z, nb * nb, b, b), 18)
    B = _rand((Z, H, nb * b, Nd), 19)
    dense = np.zeros((nb * b, nb * b))
    for k in range(nb * nb):
        r, c = divmod(k, nb)
        dense[r * b:(r + 1) * b, c * b:(c + 1) * b] = S[0, k]
    assert np.abs(oracle.dsd_t(S, B, lay, b)[0, 0] - dense.T @ B[0, 0]).max() < 1e-12


# ------------------------------------------------------------ two routes

@pytest.mark.parametrize("causal", [False, True])
def test_gradient_block_route_equals_dense_route(causal):
    Z, H, nb, b, d = 2, 2, 4, 16, 8
    lay = _layout_with_empty_row(H, nb, 20)
    Q, K, V, G = (_rand((Z, H, nb * b, d), s) for s in (21, 22, 23, 24))
    dense = oracle.attention_backward_dense(Q, K, V, G, lay, b, 0.3, causal)
    blocks = oracle.attention_backward_blocks(Q, K, V, G, lay, b, 0.3, causal)
    for x, y in zip(dense, blocks):
        assert np.abs(x - y).max() < 1e-12
    # the empty block row: no gradient reaches its queries
    assert np.all(dense[0][:, 0, b:2 * b] == 0)


# ------------------------------------------------------------ dds_t

@pytest.mark.parametrize("b", [16, 32])
def test_dds_t_is_dds_of_the_transposed_block_matrix(b):
    H, nbr, nbc, Z, M = 2, 3, 4, 2, 8
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 30 + b)
    lay[1, 2, :] = 0  # an empty block row: zero columns of the output
    nnz = int(lay.sum())
    S = _rand((Z, nnz, b, b), 31)
    A = _rand((Z, H, M, nbc * b), 32)
    layT, ST = _transposed(lay, S)
    C = oracle.dds_t(A, S, lay, b)
    assert np.abs(C - oracle.dds(A, ST, layT, b)).max() < 1e-12
    assert np.all(C[:, 1, :, 2 * b:3 * b] == 0)


def test_dds_t_all_ones_is_dense_product_with_the_transpose():
    H, nb, b, Z, M = 1, 3, 16, 1, 5
    lay = np.ones((H, nb, nb), np.uint8)
    S = _rand((Z, nb * nb, b, b), 33)
    A = _rand((Z, H, M, nb * b), 34)
    dense = np.zeros((nb * b, nb * b))
    for k in range(nb * nb):
        r, c = divmod(k, nb)
        dense[r * b:(r + 1) * b, c * b:(c + 1) * b] = S[0, k]
    assert np.abs(oracle.dds_t(A, S, lay, b)[0, 0] - A[0, 0] @ dense.T).max() < 1e-12
