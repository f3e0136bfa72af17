"""GPU parity past 32-bit element offsets: Q, K, V, O and the gradients hold
2^31 elements each (4 GiB of bf16), so every kernel's addressing of the
later heads needs 64-bit offsets. A band layout (each block row holds its
diagonal block and the one before), so that the oracle's references are
local: block row r of head h depends only on key blocks r-1 and r, and the
gradient of key block c only on query blocks c and c+1.

Inputs are drawn on the GPU from a seeded generator and the slices the
oracle needs are copied back, so both sides see the same values. About
33 GiB of device memory.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, f64, max_abs

import block_sparse_matmul_amd as bsa

pytestmark = pytest.mark.gpu

Z, H, N, B, D = 1, 256, 65536, 128, 128
NB = N // B
SCALE = 1.0 / np.sqrt(D)


def _band():
    lay = np.zeros((NB, NB), np.uint8)
    r = np.arange(NB)
    lay[r, r] = 1
    lay[r[1:], r[1:] - 1] = 1
    return lay


@pytest.fixture(scope="module")
def big():
    props = torch.cuda.get_device_properties(0)
    if props.total_memory < 48 * 2**30:
        pytest.skip("needs about 33 GiB of device memory")
    announce("64-bit offsets: bf16", Z, H, N, D)
    assert Z * H * N * D == 2**31
    g = torch.Generator(device="cuda").manual_seed(2024)
    q, k, v, do = (torch.randn((Z, H, N, D), generator=g, device="cuda", dtype=torch.bfloat16) for _ in range(4))
    lay = _band()
    L = bsa.Layout(torch.from_numpy(np.ascontiguousarray(np.broadcast_to(lay, (H, NB, NB)))), B)
    # outputs prefilled with NaN: an element no kernel writes stays NaN
    nan = lambda: torch.full((Z, H, N, D), float("nan"), device="cuda", dtype=torch.bfloat16)
    lse = torch.full((Z, H, N), float("nan"), device="cuda")
    o, lse = bsa.attention(L, q, k, v, SCALE, out=nan(), return_lse=True, lse=lse)
    dq, dk, dv = bsa.attention_backward_fused(L, q, k, v, o, lse, do, SCALE, out=(nan(), nan(), nan()))
    # the unfused chain: S holds nnz * b * b > 2^32 elements (17 GiB), then
    # the softmax in place, the DSD and a DDS on P
    s = bsa.sdd(L, q, k)
    s_blocks = {key: s[0, blk(*key)].cpu() for key in S_CASES}
    p = bsa.softmax(L, s, SCALE, inplace=True)
    o2 = bsa.dsd(L, p, v, out=nan())
    a = torch.randn((Z, H, M, N), generator=g, device="cuda", dtype=torch.bfloat16)
    c = bsa.dds(L, a, p, out=torch.full((Z, H, M, N), float("nan"), device="cuda", dtype=torch.bfloat16))
    torch.cuda.synchronize()
    yield dict(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, lay=lay, s_blocks=s_blocks, p=p, o2=o2,
               a=a, c=c)
    del q, k, v, do, o, lse, dq, dk, dv, s, p, o2, a, c
    torch.cuda.empty_cache()


M = 64  # rows of the DDS's dense operand


def blk(h, r, c):
    """Position of stored block (h, r, c) of the band layout in the block
    list (heads, then rows, then ascending columns)."""
    return h * (2 * NB - 1) + 2 * r - (c == r - 1)


def test_block_positions_follow_the_oracle_lut():
    small = 6
    lay = np.zeros((2, small, small), np.uint8)
    r = np.arange(small)
    lay[:, r, r] = 1
    lay[:, r[1:], r[1:] - 1] = 1
    lut = oracle.lut_from_layout(lay)
    pos = {}
    for h in range(2):
        for rr in range(small):
            for e in range(lut["row_ptr"][h * small + rr], lut["row_ptr"][h * small + rr + 1]):
                pos[(h, rr, int(lut["col_idx"][e]))] = e
    per_head = 2 * small - 1
    for (h, rr, cc), e in pos.items():
        assert e == h * per_head + 2 * rr - (cc == rr - 1)


S_CASES = [(0, 0, 0), (131, 256, 255), (255, 511, 510), (255, 511, 511)]


def _rows(t, h, b0, b1):
    """Token rows of blocks [b0, b1) of head h, on the CPU: [1, 1, n, D]."""
    return t[:, h:h + 1, b0 * B:b1 * B].cpu()


def test_every_output_written(big):
    for name in ("o", "lse", "dq", "dk", "dv", "o2", "c"):
        assert bool(torch.isfinite(big[name]).all()), name


@pytest.mark.parametrize("h,r,c", S_CASES)
def test_sdd_blocks(big, h, r, c):
    q, k = _rows(big["q"], h, r, r + 1), _rows(big["k"], h, c, c + 1)
    ref = oracle.sdd(q, k, np.ones((1, 1, 1), np.uint8), B)[0, 0]
    got = big["s_blocks"][(h, r, c)].double().numpy()
    assert max_abs(got, ref) <= 1e-3 * max(1.0, float(np.abs(ref).max()))


# the first and last heads (the largest offsets) and one in between; the
# first, a middle and the last block row or column
CASES = [(h, r) for h in (0, 131, H - 1) for r in (0, NB // 2, NB - 1)]


@pytest.mark.parametrize("h,r", CASES)
def test_forward_block_rows(big, h, r):
    """O and the row log-sum-exp of block row r of head h (keys r-1 and r)."""
    lo = max(r - 1, 0)
    sub = big["lay"][r:r + 1, lo:r + 1][None]
    q = _rows(big["q"], h, r, r + 1)
    k, v = _rows(big["k"], h, lo, r + 1), _rows(big["v"], h, lo, r + 1)
    ref_o = oracle.attention_dense(q, k, v, sub, B, SCALE)
    ref_l = oracle.attention_lse(q, k, sub, B, SCALE)
    assert max_abs(f64(_rows(big["o"], h, r, r + 1)), ref_o) <= TOL["bf16"]
    assert max_abs(f64(big["lse"][:, h:h + 1, r * B:(r + 1) * B].cpu()), ref_l) <= 4e-3


@pytest.mark.parametrize("h,r", CASES)
def test_backward_blocks(big, h, r):
    """dQ of block row r (keys r-1, r) and dK, dV of block column r (its
    rows r and r+1 with all their keys, r-1 .. r+1)."""
    tol = lambda ref: TOL["bf16"] * max(1.0, float(np.abs(ref).max()))
    # dQ: block row r alone
    lo = max(r - 1, 0)
    sub = big["lay"][r:r + 1, lo:r + 1][None]
    q, do = _rows(big["q"], h, r, r + 1), _rows(big["do"], h, r, r + 1)
    k, v = _rows(big["k"], h, lo, r + 1), _rows(big["v"], h, lo, r + 1)
    rdq, _, _ = oracle.attention_backward_dense(q, k, v, do, sub, B, SCALE)
    assert max_abs(f64(_rows(big["dq"], h, r, r + 1)), rdq) <= tol(rdq)
    # dK, dV: the rows that hold column r, with every key they see
    r1 = min(r + 2, NB)
    klo = max(r - 1, 0)
    khi = min(r + 2, NB)
    sub = big["lay"][r:r1, klo:khi][None]
    q, do = _rows(big["q"], h, r, r1), _rows(big["do"], h, r, r1)
    k, v = _rows(big["k"], h, klo, khi), _rows(big["v"], h, klo, khi)
    _, rdk, rdv = oracle.attention_backward_dense(q, k, v, do, sub, B, SCALE)
    c = (r - klo) * B
    for name, got, ref in (("dk", big["dk"], rdk), ("dv", big["dv"], rdv)):
        ref = ref[:, :, c:c + B]
        assert max_abs(f64(_rows(got, h, r, r + 1)), ref) <= tol(ref), name


@pytest.mark.parametrize("h,r", CASES)
def test_unfused_chain_block_rows(big, h, r):
    """Softmax blocks and DSD output of block row r (blocks r-1, r), from
    the oracle's SDD of the same inputs."""
    lo = max(r - 1, 0)
    sub = big["lay"][r:r + 1, lo:r + 1][None]
    q = _rows(big["q"], h, r, r + 1)
    k, v = _rows(big["k"], h, lo, r + 1), _rows(big["v"], h, lo, r + 1)
    ref_p = oracle.softmax(oracle.sdd(q, k, sub, B), sub, B, SCALE)
    ids = [blk(h, r, cc) for cc in range(lo, r + 1)]
    got_p = torch.stack([big["p"][0, i] for i in ids])[None].cpu()
    assert max_abs(f64(got_p), ref_p) <= 1e-4
    ref_o = oracle.dsd(f64(got_p), v, sub, B)
    assert max_abs(f64(_rows(big["o2"], h, r, r + 1)), ref_o) <= TOL["bf16"]


@pytest.mark.parametrize("h,c", CASES)
def test_dds_block_columns(big, h, c):
    """C[:, c-block] from the stored blocks of column c (rows c, c+1) and
    the matching column blocks of A."""
    r1 = min(c + 2, NB)
    sub = big["lay"][c:r1, c:c + 1][None]
    ids = [blk(h, rr, c) for rr in range(c, r1)]
    p = torch.stack([big["p"][0, i] for i in ids])[None].cpu()
    a = big["a"][:, h:h + 1, :, c * B:r1 * B].cpu()
    ref = oracle.dds(a, f64(p), sub, B)
    got = big["c"][:, h:h + 1, :, c * B:(c + 1) * B].cpu()
    assert max_abs(f64(got), ref) <= TOL["bf16"] * max(1.0, float(np.abs(ref).max()))
