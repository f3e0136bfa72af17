"""Pins for the oracle's layout -> lookup-table step and the ACSR expansion.

The layout is a tensor of 0s and 1s over non-overlapping blocks (Triton issue
117, "question on blocksparse"); ACSR is the affine-compressed row format of the
SPLAT abstract. Pins used here: a hand-worked example (tests/golden), brute
force with explicit loops, structural invariants, and a closed-form count for
the strided workload.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_lut(lay):
    """Explicit loops over every block, in the two enumeration orders."""
    H, nbr, nbc = lay.shape
    row_ptr, col_idx, ids = [0], [], {}
    for h in range(H):
        for r in range(nbr):
            for c in range(nbc):
                if lay[h, r, c]:
                    ids[(h, r, c)] = len(col_idx)
                    col_idx.append(c)
            row_ptr.append(len(col_idx))
    col_ptr, row_idx, blk_id = [0], [], []
    for h in range(H):
        for c in range(nbc):
            for r in range(nbr):
                if lay[h, r, c]:
                    row_idx.append(r)
                    blk_id.append(ids[(h, r, c)])
            col_ptr.append(len(row_idx))
    return dict(row_ptr=row_ptr, col_idx=col_idx, col_ptr=col_ptr, row_idx=row_idx, blk_id=blk_id)


def test_lut_golden_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "lut_small.json")))
    lut = oracle.lut_from_layout(np.array(g["layout"], dtype=np.uint8))
    assert int(lut["row_ptr"][-1]) == g["nnz"]
    for key in ("row_ptr", "col_idx", "col_ptr", "row_idx", "blk_id"):
        assert lut[key].tolist() == g[key], key


@pytest.mark.parametrize("shape,p,seed", [
    ((1, 1, 1), 1.0, 0), ((1, 1, 1), 0.0, 0), ((3, 5, 7), 0.4, 1), ((2, 9, 4), 0.6, 2),
    ((4, 16, 16), 0.25, 3), ((1, 33, 65), 0.1, 4), ((2, 8, 8), 0.0, 5), ((2, 8, 8), 1.0, 6),
])
def test_lut_matches_brute_force(shape, p, seed):
    lay = W.small_random_layout(*shape, p, seed)
    got = oracle.lut_from_layout(lay)
    ref = _brute_lut(lay)
    for key in ref:
        assert got[key].tolist() == ref[key], key


@pytest.mark.parametrize("idx", range(5))
def test_lut_invariants_on_workloads(idx):
    w = W.WORKLOADS[idx]
    lay = W.make_layout(w)
    H, nbr, nbc = lay.shape
    lut = oracle.lut_from_layout(lay)
    rp, ci = lut["row_ptr"], lut["col_idx"]
    cp, ri, bid = lut["col_ptr"], lut["row_idx"], lut["blk_id"]
    nnz = int(lay.sum())
    assert rp[0] == 0 and rp[-1] == nnz and np.all(np.diff(rp) >= 0)
    assert cp[0] == 0 and cp[-1] == nnz and np.all(np.diff(cp) >= 0)
    # ascending columns within each row, ascending rows within each column
    for hr in range(H * nbr):
        assert np.all(np.diff(ci[rp[hr]:rp[hr + 1]]) > 0)
    for hc in range(H * nbc):
        assert np.all(np.diff(ri[cp[hc]:cp[hc + 1]]) > 0)
    # blk_id is a permutation, and points back at the same (h, r, c)
    assert np.array_equal(np.sort(bid), np.arange(nnz))
    row_of = np.repeat(np.arange(H * nbr), np.diff(rp))
    for hc in range(H * nbc):
        h, c = divmod(hc, nbc)
        for e in range(cp[hc], cp[hc + 1]):
            k = bid[e]
            assert ci[k] == c and row_of[k] == h * nbr + ri[e]
    # dense -> LUT -> dense is the identity
    assert np.array_equal(oracle.layout_from_lut(lut, H, nbr, nbc), lay)


def test_layout_rejects_values_other_than_zero_one():
    lay = np.zeros((1, 2, 2), dtype=np.uint8)
    lay[0, 1, 1] = 2
    with pytest.raises(ValueError):
        oracle.lut_from_layout(lay)


def test_acsr_strided_equals_token_rule_quantised():
    """Expanding the strided workload's two affine terms gives exactly the
    blocks that hold at least one visible token pair of the token rule
    (brute force over every token pair of a 64x64-block grid)."""
    b, nb = 32, 64
    terms = W.strided_acsr_terms(nb, 512 // b, 128 // b)
    lay = oracle.acsr_expand(terms, 1, nb, nb)[0]
    i = np.arange(nb * b)[:, None]
    j = np.arange(nb * b)[None, :]
    tok = W.strided_token_rule(i, j, 512, 128)
    blk = tok.reshape(nb, b, nb, b).any(axis=(1, 3))
    assert np.array_equal(lay.astype(bool), blk)


def test_acsr_strided_count_closed_form():
    """Per-head block count of the strided workload (nb = 256, window 16,
    stride 4): rows r < 15 hold r + 1 window blocks, the rest 16; rows r >= 16
    add floor((r - 16) / 4) + 1 strided blocks c <= r - 16 with c = r mod 4.
    Sum: 120 + 241*16 + 4*(1 + ... + 60) = 11296."""
    nb = 256
    closed = sum(min(r + 1, 16) for r in range(nb)) + sum((r - 16) // 4 + 1 for r in range(16, nb))
    assert closed == 120 + 241 * 16 + 4 * (60 * 61 // 2) == 11296
    w = W.workload("strided_acsr_b32")
    lay = oracle.acsr_expand(W.make_acsr(w), w.H, w.nb, w.nb)
    assert lay.shape == (16, 256, 256)
    assert all(int(lay[h].sum()) == closed for h in range(w.H))
    assert np.array_equal(lay, W.make_layout(w))


def test_acsr_clipping_and_union():
    # overlapping terms union; columns outside the grid are dropped
    terms = [(0, 4, 1, -1, 1, 3), (2, 4, 0, 3, 1, 5), (1, 2, 2, 0, 0, 2)]
    lay = oracle.acsr_expand(terms, 2, 4, 5)
    ref = np.zeros((4, 5), dtype=np.uint8)
    for r in range(4):
        for c in (r - 1, r, r + 1):
            if 0 <= c < 5:
                ref[r, c] = 1
    ref[2, 3:5] = 1
    ref[3, 3:5] = 1
    ref[1, 2] = 1          # slope 2, stride 0: column 2 twice
    assert np.array_equal(lay[0], ref) and np.array_equal(lay[1], ref)
