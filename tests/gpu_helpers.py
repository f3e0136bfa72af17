"""Shared helpers of the GPU parity tests (inputs come from `workloads`,
expected values only from `oracle`)."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

# Max-abs bars for outputs of size about one (inputs N(0, 1)): fp32 1e-4;
# bf16 2e-2; fp16 5e-3. fp16 derivation: unit roundoff u = 2^-11. The
# fp16-rounded factor (P in [0, 1], or S, dS) moves each weight by at most u
# relative, so an average of values up to |v| <= 4 moves by at most about
# 2 u |v| = 3.9e-3 (the row sum uses the same rounded weights); the final
# rounding of an output below 4 adds at most 2^-10 = 9.8e-4. fp16 x fp16
# products are exact in fp32 and the fp32 accumulation adds ~1e-6.
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}


# worker threads for the oracle's full-size references (numpy releases the
# interpreter lock inside its kernels; one BLAS thread per worker)
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def pool_map(fn, chunks):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(WORKERS) as ex:
        return list(ex.map(fn, chunks))


def announce(*parts):
    """Name the case on stdout before any GPU work (flushed, so that a run
    that dies still says what it was doing)."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def to_dev(t):
    return t.contiguous().to("cuda")


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def f64(t):
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def sample_rows(layout, Z, n, seed=0):
    """Block rows (z, h, r) to check: the longest, the shortest non-empty,
    an empty one if any, and n random ones."""
    H, nbr, _ = layout.shape
    lens = layout.sum(axis=2)
    rng = np.random.default_rng(seed)
    rows = {(0, *np.unravel_index(int(np.argmax(lens)), lens.shape))}
    nz = np.argwhere(lens > 0)
    if len(nz):
        i = int(np.argmin(lens[lens > 0]))
        rows.add((Z - 1, int(nz[i][0]), int(nz[i][1])))
    empty = np.argwhere(lens == 0)
    if len(empty):
        rows.add((0, int(empty[0][0]), int(empty[0][1])))
    for _ in range(n):
        rows.add((int(rng.integers(Z)), int(rng.integers(H)), int(rng.integers(nbr))))
    return sorted((int(z), int(h), int(r)) for z, h, r in rows)


def oracle_block_sdd(q, k, layout, lut, b, z, kk):
    """S block kk of batch z by the oracle (one block, from the LUT order)."""
    H, nbr, _ = layout.shape
    hr = int(np.searchsorted(lut["row_ptr"], kk, side="right") - 1)
    h, r = divmod(hr, nbr)
    c = int(lut["col_idx"][kk])
    one = np.zeros((1, 1, 1), dtype=np.uint8)
    one[0, 0, 0] = 1
    qa = q[z:z + 1, h:h + 1, r * b:(r + 1) * b]
    ka = k[z:z + 1, h:h + 1, c * b:(c + 1) * b]
    return oracle.sdd(qa, ka, one, b)[0, 0]


def oracle_row_softmax(q, k, layout, b, scale, causal, z, h, r):
    """Softmax of one block row from the oracle's own SDD blocks:
    returns [len, b, b] in the row's block order."""
    cols = np.nonzero(layout[h, r])[0]
    sub = np.zeros((1, 1, layout.shape[2]), dtype=np.uint8)
    sub[0, 0, cols] = 1
    # the row as a one-row layout, with the query rows shifted so that the
    # causal comparison uses the true global indices
    nb = layout.shape[2]
    qa = np.zeros((1, 1, b, q.shape[3]))
    qa[0, 0] = f64(q[z, h, r * b:(r + 1) * b]) if hasattr(q, "detach") else q[z, h, r * b:(r + 1) * b]
    kf = f64(k[z:z + 1, h:h + 1]) if hasattr(k, "detach") else k[z:z + 1, h:h + 1]
    S = oracle.sdd(qa, kf, sub, b)
    if not causal:
        return oracle.softmax(S, sub, b, scale, False)[0]
    # causal on a single row: embed it at block row r of an r+1-row layout
    lay_c = np.zeros((1, r + 1, nb), dtype=np.uint8)
    lay_c[0, r, cols] = 1
    S_full = S  # the only stored blocks are those of row r
    return oracle.softmax(S_full, lay_c, b, scale, True)[0]
