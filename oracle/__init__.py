"""CPU oracle for block-sparse attention: TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy code that states what the block-sparse path
computes, written from the pages:

  * "question on blocksparse" (Triton issue 117): the three block-sparse
    matmul modes SDD (sparse = dense x dense, only the layout's blocks),
    DSD (dense = sparse x dense) and DDS (dense = dense x sparse); the layout
    as a tensor of 0s and 1s whose ones stand for 16/32/64/128-square,
    non-overlapping blocks; the SDD output in a block-sparse format that the
    block-sparse softmax and DSD reuse; that softmax reducing the rows of the
    SDD output and being the same as full-attention softmax; dense masks for
    the in-block triangle of block-triangular layouts.
  * SPLAT abstract (NSF-PAR, Jain): the affine-compressed sparse row format
    (ACSR) for regular sparse-MHSA patterns.
  * Triton tutorial, Puzzle 8 (long softmax) and Puzzle 9 (simple
    FlashAttention): the row-softmax and its streaming form.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The GPU library never does, and this package imports nothing
from it. No value computed here ever comes from the GPU path.

Conventions (readings where the pages are silent; each is listed in the
design notes):
  * layout: uint8 [H, nbr, nbc], one per head, shared across the batch.
  * block ids: the nonzero blocks enumerated in (head, block-row, block-col)
    lexicographic order; the k-th gets id k. SDD output is [Z, nnz, b, b],
    each block row-major, in that order.
  * SDD computes A @ B^T on the blocks (attention's Q K^T); DSD computes
    S @ B; DDS computes A @ S.
  * softmax applies ``scale`` to the raw SDD values, adds the optional dense
    additive masks (below), then the causal mask (-inf where the global key
    index exceeds the global query index), then a row softmax over every
    stored entry of the row. A row with no visible entry gives zeros.
  * dense masks (question on blocksparse, the answer on dense masks for
    block-triangular layouts; the page gives no format): attn_mask, float
    [Nq, Nk] over the global query and key indices, shared by every batch
    element and head, and kp_mask (key padding), float [Z, Nk] per batch
    element and key; both are added to scale * S. -inf hides an entry. Entries outside the
    layout's blocks stay hidden whatever the masks hold.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Sequence, Tuple

import numpy as np

__all__ = [
    "check_layout", "lut_from_layout", "layout_from_lut", "acsr_expand",
    "element_mask", "sdd", "softmax", "dsd", "dds",
    "attention_dense", "attention_blocks", "attention_rows", "attention_lse",
    "attention_blockrow",
    "softmax_backward", "dsd_t", "dds_t", "attention_backward_dense", "attention_backward_blocks",
]

ALLOWED_BLOCKS = (16, 32, 64, 128)


def _f64(x) -> np.ndarray:
    """Exact float64 copy of a numpy array or a (CPU) torch tensor of any
    float dtype (bf16 values are representable exactly in float64)."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# layout -> lookup tables (question on blocksparse: layout is a tensor of 0s
# and 1s, one per non-overlapping block)
# ---------------------------------------------------------------------------

def check_layout(layout) -> np.ndarray:
    """Validate a [H, nbr, nbc] layout; only 0 and 1 are allowed."""
    lay = np.asarray(layout)
    if lay.ndim != 3:
        raise ValueError("layout must be [H, nbr, nbc]")
    if not np.all((lay == 0) | (lay == 1)):
        raise ValueError("layout values must be 0 or 1")
    return lay.astype(np.uint8)


def lut_from_layout(layout) -> Dict[str, np.ndarray]:
    """Block-CSR over (h, r, c) and its CSC companion over (h, c, r).

    row_ptr[h*nbr + r] .. row_ptr[h*nbr + r + 1]: ids of the blocks of block
    row r of head h; col_idx[id] = c of that block.
    col_ptr[h*nbc + c] .. col_ptr[h*nbc + c + 1]: the blocks of block column
    c of head h in ascending r; row_idx = their r, blk_id = their CSR id.
    """
    lay = check_layout(layout)
    H, nbr, nbc = lay.shape
    hs, rs, cs = np.nonzero(lay)            # lexicographic (h, r, c)
    nnz = hs.size
    row_counts = lay.reshape(H * nbr, nbc).sum(axis=1)
    row_ptr = np.zeros(H * nbr + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(row_counts)
    col_idx = cs.astype(np.int32)

    ids = np.full(lay.shape, -1, dtype=np.int64)
    ids[hs, rs, cs] = np.arange(nnz)
    lay_t = np.transpose(lay, (0, 2, 1))    # [H, nbc, nbr]
    th, tc, tr = np.nonzero(lay_t)          # lexicographic (h, c, r)
    col_counts = lay_t.reshape(H * nbc, nbr).sum(axis=1)
    col_ptr = np.zeros(H * nbc + 1, dtype=np.int64)
    col_ptr[1:] = np.cumsum(col_counts)
    return {
        "row_ptr": row_ptr.astype(np.int32),
        "col_idx": col_idx,
        "col_ptr": col_ptr.astype(np.int32),
        "row_idx": tr.astype(np.int32),
        "blk_id": ids[th, tr, tc].astype(np.int32),
    }


def layout_from_lut(lut: Dict[str, np.ndarray], H: int, nbr: int, nbc: int) -> np.ndarray:
    """Inverse of lut_from_layout's CSR part (used by round-trip pins)."""
    lay = np.zeros((H, nbr, nbc), dtype=np.uint8)
    rp, ci = lut["row_ptr"], lut["col_idx"]
    for hr in range(H * nbr):
        h, r = divmod(hr, nbr)
        for k in range(rp[hr], rp[hr + 1]):
            lay[h, r, ci[k]] = 1
    return lay


def acsr_expand(terms: Sequence[Tuple[int, int, int, int, int, int]], H: int,
                nbr: int, nbc: int) -> np.ndarray:
    """Expand affine-compressed rows (SPLAT abstract, ACSR) to a dense layout.

    A term (row_begin, row_end, slope, offset, stride, count) puts, in every
    row r of [row_begin, row_end), the columns slope*r + offset + stride*k for
    k = 0 .. count-1 that fall inside [0, nbc). A layout is the union of its
    terms, the same for every head.
    """
    lay = np.zeros((nbr, nbc), dtype=np.uint8)
    for (r0, r1, slope, offset, stride, count) in terms:
        for r in range(max(r0, 0), min(r1, nbr)):
            for k in range(count):
                c = slope * r + offset + stride * k
                if 0 <= c < nbc:
                    lay[r, c] = 1
    return np.ascontiguousarray(np.broadcast_to(lay, (H, nbr, nbc)))


def element_mask(layout, block: int, causal: bool) -> np.ndarray:
    """Dense boolean [H, nbr*b, nbc*b]: True where a query may see a key.

    A key is visible when its block is stored, and, under the causal dense
    mask, when its global index does not exceed the query's.
    """
    lay = check_layout(layout).astype(bool)
    m = np.repeat(np.repeat(lay, block, axis=1), block, axis=2)
    if causal:
        nq, nk = m.shape[1], m.shape[2]
        m = m & (np.arange(nk)[None, None, :] <= np.arange(nq)[None, :, None])
    return m


def _bias(attn_mask, kp_mask, z: int, qi, kj) -> np.ndarray:
    """The additive dense masks at global query rows qi and key columns kj of
    batch element z: attn_mask[qi, kj] + kp_mask[z, kj] (0 for a mask that
    is None). Masks are float64 arrays here."""
    out = np.zeros((len(qi), len(kj)))
    if attn_mask is not None:
        out = out + attn_mask[np.ix_(qi, kj)]
    if kp_mask is not None:
        out = out + kp_mask[z, kj][None, :]
    return out


def _masks(attn_mask, kp_mask):
    return (None if attn_mask is None else _f64(attn_mask)), (None if kp_mask is None else _f64(kp_mask))


# ---------------------------------------------------------------------------
# the three matmul modes and the block-sparse softmax
# ---------------------------------------------------------------------------

def _blocks(layout) -> List[Tuple[int, int, int]]:
    """(h, r, c) of every stored block, in block-id order."""
    lay = check_layout(layout)
    return [tuple(int(v) for v in t) for t in zip(*np.nonzero(lay))]


def sdd(A, B, layout, block: int) -> np.ndarray:
    """Sampled dense-dense product: for block id k = (h, r, c),
    S[z, k] = A[z, h, r-block, :] @ B[z, h, c-block, :]^T."""
    A, B = _f64(A), _f64(B)
    b = block
    blocks = _blocks(layout)
    Z = A.shape[0]
    S = np.zeros((Z, len(blocks), b, b), dtype=np.float64)
    for k, (h, r, c) in enumerate(blocks):
        for z in range(Z):
            S[z, k] = A[z, h, r * b:(r + 1) * b, :] @ B[z, h, c * b:(c + 1) * b, :].T
    return S


def softmax(S, layout, block: int, scale: float, causal: bool = False, attn_mask=None,
            kp_mask=None) -> np.ndarray:
    """Block-sparse row softmax of SDD output (question on blocksparse: it
    reduces the rows of the SDD output and equals full-attention softmax).

    For query row i of block row r of head h, the row holds the entries of
    every stored block (h, r, c). x = scale*S plus the dense masks, set to
    -inf where causal hides the key, then P = exp(x - max) / sum exp(x -
    max); a row whose entries are all hidden (or that stores no block) is
    all zeros.
    """
    S = _f64(S)
    am, kpm = _masks(attn_mask, kp_mask)
    lut = lut_from_layout(layout)
    lay = check_layout(layout)
    H, nbr, _ = lay.shape
    b = block
    P = np.zeros_like(S)
    Z = S.shape[0]
    for hr in range(H * nbr):
        r = hr % nbr
        ks = list(range(lut["row_ptr"][hr], lut["row_ptr"][hr + 1]))
        if not ks:
            continue
        cols = lut["col_idx"][ks]
        qrows = r * b + np.arange(b)
        kcols = np.concatenate([c * b + np.arange(b) for c in cols])
        for z in range(Z):
            x = np.concatenate([scale * S[z, k] for k in ks], axis=1)   # [b, len*b]
            x = x + _bias(am, kpm, z, qrows, kcols)
            if causal:
                qi = r * b + np.arange(b)[:, None]
                kj = np.concatenate([c * b + np.arange(b) for c in cols])[None, :]
                x = np.where(kj <= qi, x, -np.inf)
            m = x.max(axis=1, keepdims=True)
            e = np.where(np.isfinite(m), np.exp(x - np.where(np.isfinite(m), m, 0.0)), 0.0)
            s = e.sum(axis=1, keepdims=True)
            p = np.divide(e, s, out=np.zeros_like(e), where=s > 0)
            for n, k in enumerate(ks):
                P[z, k] = p[:, n * b:(n + 1) * b]
    return P


def dsd(P, B, layout, block: int) -> np.ndarray:
    """Sparse x dense: C[z, h, r-block, :] = sum over stored (h, r, c) of
    P[z, k] @ B[z, h, c-block, :]. Rows with no stored block are zero."""
    P, B = _f64(P), _f64(B)
    lay = check_layout(layout)
    H, nbr, _ = lay.shape
    b = block
    Z, Nd = B.shape[0], B.shape[3]
    C = np.zeros((Z, H, nbr * b, Nd), dtype=np.float64)
    for k, (h, r, c) in enumerate(_blocks(lay)):
        for z in range(Z):
            C[z, h, r * b:(r + 1) * b, :] += P[z, k] @ B[z, h, c * b:(c + 1) * b, :]
    return C


def dds(A, S, layout, block: int) -> np.ndarray:
    """Dense x sparse: C[z, h, :, c-block] = sum over stored (h, r, c) of
    A[z, h, :, r-block] @ S[z, k]. Columns with no stored block are zero."""
    A, S = _f64(A), _f64(S)
    lay = check_layout(layout)
    H, _, nbc = lay.shape
    b = block
    Z, M = A.shape[0], A.shape[2]
    C = np.zeros((Z, H, M, nbc * b), dtype=np.float64)
    for k, (h, r, c) in enumerate(_blocks(lay)):
        for z in range(Z):
            C[z, h, :, c * b:(c + 1) * b] += A[z, h, :, r * b:(r + 1) * b] @ S[z, k]
    return C


def dds_t(A, S, layout, block: int) -> np.ndarray:
    """Dense x transposed sparse: C[z, h, :, r-block] = sum over stored
    (h, r, c) of A[z, h, :, c-block] @ S[z, k]^T (the DDS of the transposed
    block matrix). Block rows with no stored block give zero columns."""
    A, S = _f64(A), _f64(S)
    lay = check_layout(layout)
    H, nbr, _ = lay.shape
    b = block
    Z, M = A.shape[0], A.shape[2]
    C = np.zeros((Z, H, M, nbr * b), dtype=np.float64)
    for k, (h, r, c) in enumerate(_blocks(lay)):
        for z in range(Z):
            C[z, h, :, r * b:(r + 1) * b] += A[z, h, :, c * b:(c + 1) * b] @ S[z, k].T
    return C


# ---------------------------------------------------------------------------
# attention: two independent routes
# ---------------------------------------------------------------------------

def attention_dense(Q, K, V, layout, block: int, scale: float, causal: bool = False, attn_mask=None,
                    kp_mask=None) -> np.ndarray:
    """Route (i): dense masked attention, O = softmax(scale Q K^T + B + M) V
    with B the dense additive masks and M = 0 where element_mask is True and
    -inf elsewhere; rows with no visible key give zeros."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    am, kpm = _masks(attn_mask, kp_mask)
    mask = element_mask(layout, block, causal)
    Z, H = Q.shape[:2]
    O = np.zeros_like(Q)
    qall, kall = np.arange(Q.shape[2]), np.arange(K.shape[2])
    for z in range(Z):
        for h in range(H):
            x = scale * (Q[z, h] @ K[z, h].T)
            x = x + _bias(am, kpm, z, qall, kall)
            x = np.where(mask[h], x, -np.inf)
            m = x.max(axis=1, keepdims=True)
            ok = np.isfinite(m)
            e = np.where(ok, np.exp(x - np.where(ok, m, 0.0)), 0.0)
            s = e.sum(axis=1, keepdims=True)
            p = np.divide(e, s, out=np.zeros_like(e), where=s > 0)
            O[z, h] = p @ V[z, h]
    return O


def attention_lse(Q, K, layout, block: int, scale: float, causal: bool = False, attn_mask=None,
                  kp_mask=None) -> np.ndarray:
    """Natural log of the softmax denominator of every query row,
    log sum_j exp(x_ij) over the visible entries of x = scale Q K^T + B (the
    dense masks), [Z, H, Nq]; -inf for a row with no visible key. With it,
    P = exp(x - lse) on the visible entries (what a backward pass needs to
    rebuild P without the row max and sum)."""
    Q, K = _f64(Q), _f64(K)
    am, kpm = _masks(attn_mask, kp_mask)
    mask = element_mask(layout, block, causal)
    Z, H = Q.shape[:2]
    out = np.full(Q.shape[:3], -np.inf)
    qall, kall = np.arange(Q.shape[2]), np.arange(K.shape[2])
    for z in range(Z):
        for h in range(H):
            x = scale * (Q[z, h] @ K[z, h].T) + _bias(am, kpm, z, qall, kall)
            x = np.where(mask[h], x, -np.inf)
            m = x.max(axis=1)
            ok = np.isfinite(m)
            mm = np.where(ok, m, 0.0)
            tot = np.exp(x - mm[:, None]).sum(axis=1)   # >= 1 where ok (the max term)
            out[z, h] = np.where(ok, mm + np.log(np.where(ok, tot, 1.0)), -np.inf)
    return out


def attention_blocks(Q, K, V, layout, block: int, scale: float, causal: bool = False, attn_mask=None,
                     kp_mask=None) -> np.ndarray:
    """Route (ii): the pages' composition, SDD -> block-sparse softmax -> DSD."""
    S = sdd(Q, K, layout, block)
    P = softmax(S, layout, block, scale, causal, attn_mask, kp_mask)
    return dsd(P, V, layout, block)


def attention_blockrow(Q, K, V, layout, block: int, scale: float, causal: bool,
                       z: int, h: int, r: int) -> np.ndarray:
    """Route (ii) restricted to one block row (z, h, r): the b x d slice of O.

    Gathers the row's stored blocks, forms their SDD blocks, applies the row
    softmax across all of them and sums P-block @ V-block (DSD).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    lay = check_layout(layout)
    b = block
    cols = np.nonzero(lay[h, r])[0]
    q = Q[z, h, r * b:(r + 1) * b]
    if cols.size == 0:
        return np.zeros((b, V.shape[3]))
    s_blocks = [q @ K[z, h, c * b:(c + 1) * b].T for c in cols]
    x = scale * np.concatenate(s_blocks, axis=1)
    if causal:
        qi = r * b + np.arange(b)[:, None]
        kj = np.concatenate([c * b + np.arange(b) for c in cols])[None, :]
        x = np.where(kj <= qi, x, -np.inf)
    m = x.max(axis=1, keepdims=True)
    ok = np.isfinite(m)
    e = np.where(ok, np.exp(x - np.where(ok, m, 0.0)), 0.0)
    s = e.sum(axis=1, keepdims=True)
    p = np.divide(e, s, out=np.zeros_like(e), where=s > 0)
    out = np.zeros((b, V.shape[3]))
    for n, c in enumerate(cols):
        out += p[:, n * b:(n + 1) * b] @ V[z, h, c * b:(c + 1) * b]
    return out


def attention_rows(Q, K, V, layout, block: int, scale: float, causal: bool,
                   rows: Iterable[Tuple[int, int, int]], attn_mask=None, kp_mask=None) -> np.ndarray:
    """Route (i) on selected block rows: for each (z, h, r), the b x d slice
    of dense masked attention, computed from the full key range of head h.
    Used to check large problems on sampled outputs."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    am, kpm = _masks(attn_mask, kp_mask)
    lay = check_layout(layout)
    b = block
    out = []
    for (z, h, r) in rows:
        mask = np.repeat(lay[h, r].astype(bool), b)[None, :].repeat(b, axis=0)
        if causal:
            qi = r * b + np.arange(b)[:, None]
            mask = mask & (np.arange(mask.shape[1])[None, :] <= qi)
        x = scale * (Q[z, h, r * b:(r + 1) * b] @ K[z, h].T)
        x = x + _bias(am, kpm, z, r * b + np.arange(b), np.arange(K.shape[2]))
        x = np.where(mask, x, -np.inf)
        m = x.max(axis=1, keepdims=True)
        ok = np.isfinite(m)
        e = np.where(ok, np.exp(x - np.where(ok, m, 0.0)), 0.0)
        s = e.sum(axis=1, keepdims=True)
        p = np.divide(e, s, out=np.zeros_like(e), where=s > 0)
        out.append(p @ V[z, h])
    return np.stack(out) if out else np.zeros((0, b, V.shape[3]))


# ---------------------------------------------------------------------------
# work accounting (FLOPs over stored blocks only)
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# backward: the exact gradient of the forward, two routes
# ---------------------------------------------------------------------------
#
# The pages give the autograd pattern (Triton tutorial: a forward kernel, a
# backward kernel that receives the gradient of the output and returns the
# gradients of the inputs, both wrapped in one autograd function) and the
# three modes the attention gradient is made of. The formulas below are the
# plain calculus of O = P V with P the masked row softmax of
# X = scale Q K^T + M: for a loss L with dO = dL/dO,
#   dV = P^T dO,  dP = dO V^T,  dX = P * (dP - rowsum(P * dP)),
#   dQ = scale dX K,  dK = scale dX^T Q.
# Masked entries have P = 0 and so get no gradient.


def softmax_backward(P, dP, layout, block: int, scale: float) -> np.ndarray:
    """Gradient of the block-sparse softmax with respect to its input S,
    given its output P and the gradient dP of the output: for each query
    row, D = sum over the row's stored entries of P * dP, and
    dS = scale * P * (dP - D). Entries the mask hid (P = 0) get zero."""
    P, dP = _f64(P), _f64(dP)
    lut = lut_from_layout(layout)
    lay = check_layout(layout)
    H, nbr, _ = lay.shape
    dS = np.zeros_like(P)
    for hr in range(H * nbr):
        ks = list(range(lut["row_ptr"][hr], lut["row_ptr"][hr + 1]))
        if not ks:
            continue
        for z in range(P.shape[0]):
            D = sum((P[z, k] * dP[z, k]).sum(axis=1, keepdims=True) for k in ks)   # [b, 1]
            for k in ks:
                dS[z, k] = scale * P[z, k] * (dP[z, k] - D)
    return dS


def dsd_t(S, B, layout, block: int) -> np.ndarray:
    """Transposed sparse x dense: C[z, h, c-block, :] = sum over stored
    (h, r, c) of S[z, k]^T @ B[z, h, r-block, :] (the DSD of the transposed
    block matrix; in attention's backward dK = dS^T Q and dV = P^T dO).
    Block columns with no stored block give zero rows."""
    S, B = _f64(S), _f64(B)
    lay = check_layout(layout)
    H, _, nbc = lay.shape
    b = block
    Z, Nd = B.shape[0], B.shape[3]
    C = np.zeros((Z, H, nbc * b, Nd), dtype=np.float64)
    for k, (h, r, c) in enumerate(_blocks(lay)):
        for z in range(Z):
            C[z, h, c * b:(c + 1) * b, :] += S[z, k].T @ B[z, h, r * b:(r + 1) * b, :]
    return C


def attention_backward_dense(Q, K, V, dO, layout, block: int, scale: float, causal: bool = False, attn_mask=None,
                             kp_mask=None):
    """Route (i) of the gradient: dense matrices with the element mask.
    Returns (dQ, dK, dV) for the forward of attention_dense (the additive
    masks are constants: they shape P and get no gradient)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    am, kpm = _masks(attn_mask, kp_mask)
    mask = element_mask(layout, block, causal)
    Z, H = Q.shape[:2]
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    qall, kall = np.arange(Q.shape[2]), np.arange(K.shape[2])
    for z in range(Z):
        for h in range(H):
            x = scale * (Q[z, h] @ K[z, h].T) + _bias(am, kpm, z, qall, kall)
            x = np.where(mask[h], x, -np.inf)
            m = x.max(axis=1, keepdims=True)
            e = np.where(np.isfinite(m), np.exp(x - np.where(np.isfinite(m), m, 0.0)), 0.0)
            s = e.sum(axis=1, keepdims=True)
            P = np.divide(e, s, out=np.zeros_like(e), where=s > 0)
            dV[z, h] = P.T @ dO[z, h]
            dP = dO[z, h] @ V[z, h].T
            dX = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dQ[z, h] = scale * (dX @ K[z, h])
            dK[z, h] = scale * (dX.T @ Q[z, h])
    return dQ, dK, dV


def attention_backward_blocks(Q, K, V, dO, layout, block: int, scale: float, causal: bool = False, attn_mask=None,
                              kp_mask=None):
    """Route (ii) of the gradient, on the block-sparse operators: P by SDD
    and softmax (recomputed), dP = SDD(dO, V), dS = softmax_backward(P, dP),
    dQ = DSD(dS, K), dK = DSD^T(dS, Q), dV = DSD^T(P, dO)."""
    P = softmax(sdd(Q, K, layout, block), layout, block, scale, causal, attn_mask, kp_mask)
    dS = softmax_backward(P, sdd(dO, V, layout, block), layout, block, scale)
    return dsd(dS, K, layout, block), dsd_t(dS, Q, layout, block), dsd_t(P, dO, layout, block)

