"""Pins for the oracle's dense additive masks (question on blocksparse: dense
masks can be passed alongside the layout; the page gives no format, and
the one taken here is: attn_mask [Nq, Nk] shared by batch and heads,
kp_mask [Z, Nk] per batch element, both added to scale * S).

Independent routes: torch's scaled_dot_product_attention math path in
float64 with a float (additive) attn_mask, forward and autograd; attention
over truncated key sequences for key padding; the causal flag against the
same triangle as an additive mask; the layout against the same pattern as
an additive mask on an all-ones layout; shift invariance of the softmax
under a per-row constant; finite differences of the masked forward.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(Q, K, V, bias, scale):
    """torch SDPA (math backend, float64) with an additive float mask."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    q, k, v = (torch.tensor(x) for x in (Q, K, V))
    with sdpa_kernel(SDPBackend.MATH):
        return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.tensor(bias),
                                                                scale=scale).numpy()


def test_additive_masks_are_sdpa_float_mask_on_all_ones_layout():
    """Finite masks: the bias SDPA adds is attn_mask[i, j] + kp_mask[z, j]."""
    Z, H, nb, b, d = 2, 3, 3, 16, 8
    N = nb * b
    lay = np.ones((H, nb, nb), np.uint8)
    Q, K, V = (_rand((Z, H, N, d), s) for s in (1, 2, 3))
    am = _rand((N, N), 4)
    kp = _rand((Z, N), 5) * 2
    bias = am[None, None] + kp[:, None, None, :]
    ref = _sdpa(Q, K, V, bias, 0.3)
    assert np.abs(oracle.attention_dense(Q, K, V, lay, b, 0.3, False, am, kp) - ref).max() < 1e-12
    assert np.abs(oracle.attention_blocks(Q, K, V, lay, b, 0.3, False, am, kp) - ref).max() < 1e-12


def test_key_padding_is_attention_over_the_truncated_keys():
    """kp_mask = -inf beyond the first n_z keys of batch element z gives the
    unmasked attention over those n_z keys (SDPA on the truncated
    sequences); lengths that are not multiples of the block included."""
    Z, H, nb, b, d = 3, 2, 4, 16, 8
    N = nb * b
    lay = np.ones((H, nb, nb), np.uint8)
    Q, K, V = (_rand((Z, H, N, d), s) for s in (6, 7, 8))
    lens = [N, 37, 5]
    kp = np.zeros((Z, N))
    for z, n in enumerate(lens):
        kp[z, n:] = -np.inf
    O = oracle.attention_dense(Q, K, V, lay, b, 0.25, False, kp_mask=kp)
    for z, n in enumerate(lens):
        ref = _sdpa(Q[z:z + 1], K[z:z + 1, :, :n], V[z:z + 1, :, :n], np.zeros((N, n)), 0.25)
        assert np.abs(O[z:z + 1] - ref).max() < 1e-12, z


def test_additive_triangle_equals_causal_flag():
    """-inf above the diagonal as attn_mask, causal off, equals the causal
    flag (a mask read with query and key swapped would not)."""
    Z, H, nb, b, d = 2, 2, 4, 16, 8
    N = nb * b
    lay = W.small_random_layout(H, nb, nb, 0.6, 9, force_diagonal=True)
    Q, K, V = (_rand((Z, H, N, d), s) for s in (10, 11, 12))
    tri = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], 0.0, -np.inf)
    ref = oracle.attention_dense(Q, K, V, lay, b, 0.5, True)
    assert np.abs(oracle.attention_dense(Q, K, V, lay, b, 0.5, False, tri) - ref).max() < 1e-12
    S = oracle.sdd(Q, K, lay, b)
    assert np.abs(oracle.softmax(S, lay, b, 0.5, False, tri) - oracle.softmax(S, lay, b, 0.5, True)).max() < 1e-12


def test_layout_as_additive_mask_on_all_ones_layout():
    """A block pattern given as an additive mask on the all-ones layout
    equals the block-sparse attention with that pattern as the layout (on a
    non-square grid, so a transposed mask cannot line up)."""
    Z, H, nbr, nbc, b, d = 2, 1, 3, 5, 16, 8
    lay = W.small_random_layout(H, nbr, nbc, 0.5, 13)
    lay[0, :, 0] = 1  # every row sees something
    Q = _rand((Z, H, nbr * b, d), 14)
    K, V = _rand((Z, H, nbc * b, d), 15), _rand((Z, H, nbc * b, d), 16)
    am = np.where(oracle.element_mask(lay, b, False)[0], 0.0, -np.inf)
    ones = np.ones((H, nbr, nbc), np.uint8)
    ref = oracle.attention_dense(Q, K, V, lay, b, 0.4)
    assert np.abs(oracle.attention_dense(Q, K, V, ones, b, 0.4, False, am) - ref).max() < 1e-12
    assert np.abs(oracle.attention_blocks(Q, K, V, ones, b, 0.4, False, am) - ref).max() < 1e-12


def test_row_constant_mask_changes_nothing():
    """softmax(x + c_i) = softmax(x) for a constant per query row."""
    Z, H, nb, b = 2, 2, 3, 16
    N = nb * b
    lay = W.small_random_layout(H, nb, nb, 0.6, 17, force_diagonal=True)
    S = _rand((Z, int(lay.sum()), b, b), 18)
    c = _rand((N, 1), 19) * 50
    P0 = oracle.softmax(S, lay, b, 0.7, True)
    assert np.abs(oracle.softmax(S, lay, b, 0.7, True, np.repeat(c, N, axis=1)) - P0).max() < 1e-12


def test_fully_masked_rows_are_zero_and_masked_entries_get_zero():
    Z, H, nb, b, d = 2, 2, 3, 16, 8
    N = nb * b
    lay = np.ones((H, nb, nb), np.uint8)
    Q, K, V = (_rand((Z, H, N, d), s) for s in (20, 21, 22))
    am = _rand((N, N), 23)
    am[5, :] = -np.inf       # query 5 sees nothing
    am[7, 3] = -np.inf       # one entry hidden
    kp = np.zeros((Z, N))
    kp[1, :] = -np.inf       # batch element 1 sees nothing at all
    O = oracle.attention_dense(Q, K, V, lay, b, 0.3, False, am, kp)
    assert np.all(O[:, :, 5] == 0) and np.all(O[1] == 0)
    S = oracle.sdd(Q, K, lay, b)
    P = oracle.softmax(S, lay, b, 0.3, False, am, kp)
    lut = oracle.lut_from_layout(lay)
    k0 = int(lut["row_ptr"][0])  # head 0, block row 0 holds query 7; key 3 is in its first block
    assert P[0, k0, 7, 3] == 0 and np.all(P[1] == 0)
    assert not np.isnan(P).any()


@pytest.mark.parametrize("causal", [False, True])
def test_masked_gradient_is_sdpa_autograd(causal):
    Z, H, nb, b, d = 2, 2, 3, 16, 8
    N = nb * b
    lay = np.ones((H, nb, nb), np.uint8)
    Q, K, V, G = (_rand((Z, H, N, d), s) for s in (24, 25, 26, 27))
    am = _rand((N, N), 28)
    kp = np.zeros((Z, N))
    kp[0, 40:] = -np.inf
    bias = am[None, None] + kp[:, None, None, :]
    if causal:
        bias = bias + np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], 0.0, -np.inf)
    dQ, dK, dV = oracle.attention_backward_dense(Q, K, V, G, lay, b, 0.35, causal, am, kp)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    from torch.nn.attention import SDPBackend, sdpa_kernel
    with sdpa_kernel(SDPBackend.MATH):
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.tensor(bias), scale=0.35)
    o.backward(torch.tensor(G))
    for name, ours, ref in (("Q", dQ, q.grad), ("K", dK, k.grad), ("V", dV, v.grad)):
        assert np.abs(ours - ref.numpy()).max() < 1e-10, name
    blocks = oracle.attention_backward_blocks(Q, K, V, G, lay, b, 0.35, causal, am, kp)
    for x, y in zip((dQ, dK, dV), blocks):
        assert np.abs(x - y).max() < 1e-12


def test_masked_rows_route_equals_dense_route():
    Z, H, nb, b, d = 2, 2, 4, 16, 8
    N = nb * b
    lay = W.small_random_layout(H, nb, nb, 0.5, 29, force_diagonal=True)
    Q, K, V = (_rand((Z, H, N, d), s) for s in (30, 31, 32))
    am = _rand((N, N), 33)
    kp = _rand((Z, N), 34)
    rows = [(0, 0, 0), (1, 1, 3), (0, 1, 2)]
    dense = oracle.attention_dense(Q, K, V, lay, b, 0.3, True, am, kp)
    got = oracle.attention_rows(Q, K, V, lay, b, 0.3, True, rows, am, kp)
    for n, (z, h, r) in enumerate(rows):
        assert np.abs(got[n] - dense[z, h, r * b:(r + 1) * b]).max() < 1e-12


# ------------------------------------------------------------ row log-sum-exp

def test_lse_all_ones_is_torch_logsumexp():
    Z, H, nb, b, d = 2, 2, 3, 16, 8
    N = nb * b
    lay = np.ones((H, nb, nb), np.uint8)
    Q, K = _rand((Z, H, N, d), 40), _rand((Z, H, N, d), 41)
    am = _rand((N, N), 42)
    ref = torch.logsumexp(torch.tensor(0.3 * (Q @ np.swapaxes(K, 2, 3)) + am), dim=-1).numpy()
    assert np.abs(oracle.attention_lse(Q, K, lay, b, 0.3, False, am) - ref).max() < 1e-12


def test_lse_rebuilds_p_and_the_output():
    """exp(x - lse) over the visible entries sums to one per row and, times
    V, gives the attention output; an empty row has lse = -inf; under causal
    the first query sees only key 0, so its lse is that one score."""
    Z, H, nb, b, d = 2, 2, 4, 16, 8
    N = nb * b
    lay = W.small_random_layout(H, nb, nb, 0.5, 43, force_diagonal=True)
    lay[1, 2, :] = 0
    Q, K, V = (_rand((Z, H, N, d), s) for s in (44, 45, 46))
    kp = _rand((Z, N), 47)
    lse = oracle.attention_lse(Q, K, lay, b, 0.4, True, kp_mask=kp)
    mask = oracle.element_mask(lay, b, True)
    O = oracle.attention_dense(Q, K, V, lay, b, 0.4, True, kp_mask=kp)
    for z in range(Z):
        for h in range(H):
            x = 0.4 * Q[z, h] @ K[z, h].T + kp[z][None, :]
            ok = np.isfinite(lse[z, h])
            P = np.where(mask[h] & ok[:, None], np.exp(x - np.where(ok, lse[z, h], 0.0)[:, None]), 0.0)
            assert np.abs(P.sum(axis=1) - ok).max() < 1e-12
            assert np.abs(P @ V[z, h] - O[z, h]).max() < 1e-12
    assert np.all(np.isneginf(lse[:, 1, 2 * b:3 * b]))
    assert np.abs(lse[:, :, 0] - (0.4 * (Q[:, :, 0] * K[:, :, 0]).sum(-1) + kp[:, None, 0])).max() < 1e-12
