"""The fused attention that shares K/V across block rows (slope-1 ACSR
layouts; float32 kernel and the 16-bit kernel's sharing mode): groups of
rows r0, r0 + t, ... walk the union of their columns and stage each block
once. Parity against the oracle's dense route
on small layouts whose groups are ragged (rows past the grid, columns held by
one row only, rows with no block at all), causal and not, blocks of 32 and
64, head_dim 64 and 128; the row log-sum-exp; agreement with the one-row
kernel on the same handle; the plan the handle reports against the rule it
states (two rows a workgroup, at the row stride whose shifted offset sets
have the smallest union, kept when the rows hold at least 1.5 times as many
blocks as the union). Sharing is off by default and turned on here.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, f64, max_abs, to_dev

import block_sparse_matmul_amd as bsa

pytestmark = pytest.mark.gpu


def _offsets(terms, nbr, nbc):
    """Relative offsets of slope-1 terms covering every row, on the grid."""
    d = set()
    for (_, _, _, off, stride, count) in terms:
        for k in range(count):
            v = off + stride * k
            if -(nbr - 1) <= v <= nbc - 1:
                d.add(v)
    return sorted(d)


def _expected_plan(terms, nb, block):
    G = 2
    d = _offsets(terms, nb, nb)
    if block < 32 or nb < 2 or not d:
        return (1, 0)
    best = None
    for t in range(1, min(64, (nb - 1) // (G - 1)) + 1):
        n = len({o + j * t for o in d for j in range(G)})
        if best is None or n < best[1]:
            best = (t, n)
    if best is None or 3 * best[1] > 2 * G * len(d):
        return (1, 0)
    return (G, best[0])


# (terms, nb): local window + stride 4 (the strided workload's shape, small);
# a window alone on a grid the groups do not divide; a window reaching three
# blocks ahead (causal cuts it); offsets 2..4 only (the last rows are empty,
# and causal empties every row); overlapping terms with offsets beyond the
# grid and a negative stride
CASES = [
    ([(0, 40, 1, -5, 1, 6), (0, 40, 1, -40, 4, 11)], 40),
    ([(0, 37, 1, -7, 1, 8)], 37),
    ([(0, 23, 1, -3, 1, 7)], 23),
    ([(0, 14, 1, 2, 1, 3)], 14),
    ([(0, 19, 1, -30, 1, 33), (0, 19, 1, 4, -3, 3)], 19),
]
SHAPES = [(32, 64), (32, 128), (64, 64)]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("shape", SHAPES, ids=[f"b{b}d{d}" for b, d in SHAPES])
@pytest.mark.parametrize("causal", [False, True])
def test_band_attention_matches_oracle(case, shape, causal):
    terms, nb = CASES[case]
    b, d = shape
    H, Z = 2, 2
    announce("band attention", case, b, d, causal)
    lay = oracle.acsr_expand(terms, H, nb, nb)
    g = torch.Generator("cpu").manual_seed(700 + case)
    q, k, v = (torch.randn((Z, H, nb * b, d), generator=g) for _ in range(3))
    L = bsa.Layout.acsr(terms, H, nb, nb, b)
    plan = L.kv_share()
    assert plan == _expected_plan(terms, nb, b) and plan[0] == 2
    L.set_kv_share(True)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    O, lse = bsa.attention(L, qd, kd, vd, 0.125, causal, return_lse=True,
                           out=torch.full_like(qd, float("nan")))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all()), "unwritten output"
    ref = oracle.attention_dense(q, k, v, lay, b, 0.125, causal)
    assert max_abs(f64(O), ref) <= TOL["f32"]
    ref_lse = oracle.attention_lse(q, k, lay, b, 0.125, causal)
    got = f64(lse)
    inf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got), inf)
    if (~inf).any():
        assert float(np.abs(got[~inf] - ref_lse[~inf]).max()) <= TOL["f32"]
    # the one-row kernel on the same handle
    L.set_kv_share(False)
    O1 = bsa.attention(L, qd, kd, vd, 0.125, causal)
    assert max_abs(f64(O), f64(O1)) <= 1e-5


def test_band_plans_of_the_cases():
    """The plans the handles report: the rule above for every case at
    every block (none at blocks of 16), the strided workload's shape on
    stride 4, and no plan where no shift overlaps enough (offsets -10, 0,
    7: any shift keeps at most one of the three)."""
    announce("band plans")
    sparse = ([(0, 12, 1, -10, 10, 2), (0, 12, 1, 7, 1, 1)], 12)
    for terms, nb in CASES + [sparse]:
        for b in (16, 32, 64, 128):
            assert bsa.Layout.acsr(terms, 1, nb, nb, b).kv_share() == _expected_plan(terms, nb, b), (terms, b)
    assert bsa.Layout.acsr(CASES[0][0], 1, 40, 40, 32).kv_share() == (2, 4)
    assert bsa.Layout.acsr(sparse[0], 1, 12, 12, 32).kv_share() == (1, 0)


def test_band_switch():
    announce("band switch")
    terms, nb = CASES[0]
    L = bsa.Layout.acsr(terms, 1, nb, nb, 32)
    for bad in (2, -2):
        assert bsa._lib.lib().bs_layout_set_kv_share(L.handle, bad) == bsa._lib.BS_ERR_INVALID_ARG
    L.set_kv_share(True)
    L.set_kv_share(False)
    assert L.kv_share() == (2, 4)  # the plan stays; only its use is off
    L.set_kv_share(None)


@pytest.mark.parametrize("b,dt,shares", [(32, "f32", False), (64, "bf16", True), (128, "bf16", False)])
def test_band_default_mode(b, dt, shares):
    """The default (-1): the sharing kernel for 16-bit operands with blocks
    of 64, the one-row kernel otherwise; each gives the same bits as the
    kernel forced on or off (the small cases here run one key group per row
    where sharing is off, so both give the same bits anyway for float32)."""
    terms, nb = CASES[0]
    H, Z, d = 2, 1, 64
    announce("band default mode", b, dt)
    g = torch.Generator("cpu").manual_seed(790 + b)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    q, k, v = (to_dev(torch.randn((Z, H, nb * b, d), generator=g).to(tdt)) for _ in range(3))
    L = bsa.Layout.acsr(terms, H, nb, nb, b)
    O_def = bsa.attention(L, q, k, v, 0.125)
    L.set_kv_share(shares)
    O_forced = bsa.attention(L, q, k, v, 0.125)
    assert torch.equal(O_def, O_forced)


@pytest.mark.parametrize("b,dt", [(32, "f32"), (64, "f32"), (32, "bf16"), (64, "bf16"), (128, "bf16")])
def test_band_attention_non_square(b, dt):
    """More key blocks than query blocks (the terms reach past the last
    row's diagonal): the plan clips columns at the key grid."""
    terms = [(0, 20, 1, -3, 1, 12), (0, 20, 1, -20, 4, 12)]
    nbr, nbc, H, Z, d = 20, 28, 2, 2, 64
    announce("band attention non-square", b, dt)
    lay = oracle.acsr_expand(terms, H, nbr, nbc)
    g = torch.Generator("cpu").manual_seed(760 + b)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    q = torch.randn((Z, H, nbr * b, d), generator=g).to(tdt)
    k, v = (torch.randn((Z, H, nbc * b, d), generator=g).to(tdt) for _ in range(2))
    L = bsa.Layout.acsr(terms, H, nbr, nbc, b)
    assert L.kv_share()[0] == 2
    L.set_kv_share(True)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    O = bsa.attention(L, qd, kd, vd, 0.125, out=torch.full_like(qd, float("nan")))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all())
    assert max_abs(f64(O), oracle.attention_dense(q, k, v, lay, b, 0.125)) <= TOL[dt]


WIDE_SHAPES = [(32, 64), (32, 128), (64, 128), (128, 64), (128, 128)]
DT16 = {"bf16": torch.bfloat16, "f16": torch.float16}
LSE_TOL16 = {"bf16": 4e-3, "f16": 1e-3}


@pytest.mark.parametrize("case", [0, 1, 3, 4])
@pytest.mark.parametrize("shape", WIDE_SHAPES, ids=[f"b{b}d{d}" for b, d in WIDE_SHAPES])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_band_attention_16bit_matches_oracle(case, shape, dt, causal):
    """The 16-bit kernel with K/V shared across two rows: the oracle on the
    rounded inputs at the 16-bit bars, the row log-sum-exp, and the same
    kernel without sharing on the same handle."""
    terms, nb = CASES[case]
    b, d = shape
    H, Z = 2, 2
    announce("band attention 16-bit", case, b, d, dt, causal)
    lay = oracle.acsr_expand(terms, H, nb, nb)
    g = torch.Generator("cpu").manual_seed(780 + case)
    q, k, v = (torch.randn((Z, H, nb * b, d), generator=g).to(DT16[dt]) for _ in range(3))
    L = bsa.Layout.acsr(terms, H, nb, nb, b)
    assert L.kv_share()[0] == 2
    L.set_kv_share(True)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    O, lse = bsa.attention(L, qd, kd, vd, 0.125, causal, return_lse=True, out=torch.full_like(qd, float("nan")))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all()), "unwritten output"
    ref = oracle.attention_dense(q, k, v, lay, b, 0.125, causal)
    assert max_abs(f64(O), ref) <= TOL[dt]
    ref_lse = oracle.attention_lse(q, k, lay, b, 0.125, causal)
    got = f64(lse)
    inf = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(got), inf)
    if (~inf).any():
        assert float(np.abs(got[~inf] - ref_lse[~inf]).max()) <= LSE_TOL16[dt]
    L.set_kv_share(False)
    O1 = bsa.attention(L, qd, kd, vd, 0.125, causal)
    assert max_abs(f64(O), f64(O1)) <= TOL[dt]


def test_band_layout_with_masks_takes_the_masked_kernel():
    """A sharing plan does not apply with dense masks: the masked kernel
    runs (sharing forced on or not) and matches the oracle."""
    terms, nb = CASES[0]
    b, d, H, Z = 64, 64, 2, 2
    N = nb * b
    announce("band layout with masks")
    lay = oracle.acsr_expand(terms, H, nb, nb)
    g = torch.Generator("cpu").manual_seed(800)
    q, k, v = (torch.randn((Z, H, N, d), generator=g).to(torch.bfloat16) for _ in range(3))
    kp = torch.randn((Z, N), generator=g)
    kp[1, N // 3:] = -float("inf")
    L = bsa.Layout.acsr(terms, H, nb, nb, b)
    ref = oracle.attention_dense(q, k, v, lay, b, 0.125, False, kp_mask=kp)
    for mode in (None, True, False):
        L.set_kv_share(mode)
        O = bsa.attention(L, to_dev(q), to_dev(k), to_dev(v), 0.125, key_padding_mask=to_dev(kp))
        assert max_abs(f64(O), ref) <= TOL["bf16"], mode
