"""Seeded synthetic inputs for block-sparse attention.

This module is shared by the CPU oracle, the tests and the benchmark. It holds
no arithmetic of the method itself: it only draws 0/1 block layouts (and, for
the strided pattern, the affine terms that describe it) and random tensors.

Layouts follow the patterns the pages name for sparse multi-head attention:
a causal block-triangular layout (question on blocksparse, answer on dense
masks), BigBird-style window + global + random blocks at 64x64 (same page,
BigBird question), a Sparse-Transformer-style local+strided pattern described
by affine row terms (SPLAT abstract, ACSR) and a large random layout in the
moderate 10-50% density band the SPLAT abstract gives.

Randomness:
  * layouts: ``numpy.random.default_rng(seed)``
  * tensors: ``torch.Generator('cpu').manual_seed(seed)``, drawn in the order
    Q, K, V, then the dense DDS operand, as float32 N(0, 1); bf16 workloads
    round those float32 draws to bfloat16 (round-to-nearest-even).
Everything is produced on the CPU so that the oracle and the GPU path see the
same values.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

# One affine row term: rows [row_begin, row_end) hold the columns
# slope*r + offset + stride*k for k in [0, count), clipped to the grid.
AcsrTerm = Tuple[int, int, int, int, int, int]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    Z: int          # batch
    H: int          # heads
    N: int          # sequence length (queries = keys)
    d: int          # head dimension
    block: int      # block edge (16, 32, 64 or 128)
    dtype: str      # "f32" or "bf16"
    causal: bool    # in-block causal mask on top of the block layout
    pattern: str    # generator name, see make_layout
    dds_m: int = 0  # rows of the dense operand of the standalone DDS (0: none)

    @property
    def nb(self) -> int:
        return self.N // self.block

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


# The five workloads: tiny, causal block-triangular, BigBird, strided (ACSR)
# with a standalone DDS, and large random in bf16.
WORKLOADS: List[Workload] = [
    Workload("tiny_b16", 1, 1, 256, 64, 16, "f32", False, "random_p0.3"),
    Workload("causal_b64", 4, 12, 2048, 64, 64, "f32", True, "lower_triangular"),
    Workload("bigbird_b64", 2, 16, 4096, 64, 64, "f32", False, "bigbird"),
    Workload("strided_acsr_b32", 1, 16, 8192, 64, 32, "f32", False, "strided_acsr", dds_m=64),
    Workload("random_b128_bf16", 1, 32, 16384, 128, 128, "bf16", False, "random_p0.25_per_head"),
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


# --------------------------------------------------------------------------
# layouts
# --------------------------------------------------------------------------

def random_layout(H: int, nb: int, p: float, rng: np.random.Generator,
                  force_diagonal: bool = True) -> np.ndarray:
    """Each block on with probability p (independent per head), diagonal on."""
    lay = (rng.random((H, nb, nb)) < p).astype(np.uint8)
    if force_diagonal:
        idx = np.arange(nb)
        lay[:, idx, idx] = 1
    return lay


def lower_triangular_layout(H: int, nb: int) -> np.ndarray:
    """Block (r, c) on iff c <= r, the same for every head."""
    tri = np.tril(np.ones((nb, nb), dtype=np.uint8))
    return np.ascontiguousarray(np.broadcast_to(tri, (H, nb, nb)))


def bigbird_layout(H: int, nb: int, rng: np.random.Generator, window: int = 1,
                   n_global: int = 2, n_random: int = 3) -> np.ndarray:
    """Sliding window of 2*window+1 blocks, the first n_global block rows and
    columns fully on, and n_random uniformly drawn blocks per block row
    (drawn per head, head-major then row order; they may coincide with the
    window or global blocks)."""
    lay = np.zeros((H, nb, nb), dtype=np.uint8)
    for h in range(H):
        for r in range(nb):
            lo, hi = max(0, r - window), min(nb, r + window + 1)
            lay[h, r, lo:hi] = 1
        lay[h, :n_global, :] = 1
        lay[h, :, :n_global] = 1
        for r in range(nb):
            cols = rng.choice(nb, n_random, replace=False)
            lay[h, r, cols] = 1
    return lay


def strided_acsr_terms(nb: int, window_blocks: int, stride_blocks: int) -> List[AcsrTerm]:
    """Affine terms of the causal local + strided pattern at block level.

    Term 1: the window c in [r - window_blocks + 1, r].
    Term 2: every stride_blocks-th block counting back from the diagonal,
            c = r - stride_blocks*k for k >= 0 (written as an ascending run
            starting at r - nb with the count that reaches c = r).
    Columns outside [0, nb) are clipped away by the format itself.
    """
    assert nb % stride_blocks == 0
    t1 = (0, nb, 1, -(window_blocks - 1), 1, window_blocks)
    t2 = (0, nb, 1, -nb, stride_blocks, nb // stride_blocks + 1)
    return [t1, t2]


def strided_token_rule(i: np.ndarray, j: np.ndarray, window_tokens: int,
                       stride_tokens: int) -> np.ndarray:
    """Token-level pattern the strided workload quantises: key j visible to
    query i iff j <= i and (i - j < window or (i - j) % stride == 0)."""
    diff = i - j
    return (diff >= 0) & ((diff < window_tokens) | (diff % stride_tokens == 0))


def make_layout(w: Workload, seed: int = 0) -> np.ndarray:
    """Dense uint8 [H, nb, nb] layout of a workload (seeded)."""
    rng = np.random.default_rng(seed)
    nb = w.nb
    if w.pattern == "random_p0.3":
        return random_layout(w.H, nb, 0.3, rng)
    if w.pattern == "lower_triangular":
        return lower_triangular_layout(w.H, nb)
    if w.pattern == "bigbird":
        return bigbird_layout(w.H, nb, rng)
    if w.pattern == "strided_acsr":
        # Dense form of the same pattern, evaluated at block level from the
        # token rule: a block is on iff some token pair inside it is.
        r = np.arange(nb)[:, None]
        c = np.arange(nb)[None, :]
        diff = r - c
        wb, sb = 512 // w.block, 128 // w.block
        blk = (diff >= 0) & ((diff <= wb) | (diff % sb == 0))
        return np.ascontiguousarray(np.broadcast_to(blk.astype(np.uint8), (w.H, nb, nb)))
    if w.pattern == "random_p0.25_per_head":
        return random_layout(w.H, nb, 0.25, rng)
    raise ValueError(w.pattern)


def make_acsr(w: Workload) -> Optional[List[AcsrTerm]]:
    """Affine terms for workloads stored in ACSR (None for the others)."""
    if w.pattern != "strided_acsr":
        return None
    return strided_acsr_terms(w.nb, 512 // w.block, 128 // w.block)


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------

def make_qkv(w: Workload, seed: int = 0):
    """CPU tensors Q, K, V of shape [Z, H, N, d] (float32 or bfloat16)."""
    import torch
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (w.Z, w.H, w.N, w.d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if w.dtype == "bf16":
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    return q, k, v


def make_dense(shape, seed: int, dtype: str = "f32", after: int = 0):
    """N(0,1) float32 tensor (optionally rounded to bf16). ``after`` draws are
    skipped first so that e.g. the DDS operand follows Q, K, V in one stream."""
    import torch
    g = torch.Generator("cpu").manual_seed(seed)
    if after:
        torch.randn((after,), generator=g, dtype=torch.float32)
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t


def make_dds_operands(w: Workload, nnz: int, seed: int = 0):
    """Inputs of the standalone DDS: dense A [Z, H, M, N] N(0,1), drawn after
    Q, K, V in the same stream, and block values S [Z, nnz, b, b] drawn
    U[0, 1) / (8 b) from a second stream (probability-like magnitudes, as the
    softmax output the DDS consumes in attention)."""
    import torch
    m = w.dds_m
    n_qkv = 3 * w.Z * w.H * w.N * w.d
    a = make_dense((w.Z, w.H, m, w.N), seed, "f32", after=n_qkv)
    g = torch.Generator("cpu").manual_seed(seed + 1)
    s = torch.rand((w.Z, nnz, w.block, w.block), generator=g, dtype=torch.float32)
    s = s / (8.0 * w.block)
    if w.dtype == "bf16":
        a = a.to(torch.bfloat16)
    return a, s


def small_random_layout(H: int, nbr: int, nbc: int, p: float, seed: int,
                        force_diagonal: bool = False) -> np.ndarray:
    """Random 0/1 layout of any shape (for sweeps and edge cases)."""
    rng = np.random.default_rng(seed)
    lay = (rng.random((H, nbr, nbc)) < p).astype(np.uint8)
    if force_diagonal:
        n = min(nbr, nbc)
        lay[:, np.arange(n), np.arange(n)] = 1
    return lay
