"""Block-sparse multi-head attention for AMD MI355X (gfx950).

Python binding of libbsattn.so (include/bsattn.h): argument checks and
marshalling only; every step runs in the library's HIP kernels. PyTorch
supplies device memory and the current stream.

    L = Layout(layout_uint8[H, nbr, nbc], block)        # or Layout.acsr(...)
    S = sdd(L, q, k)                  # [Z, nnz, b, b] float32, S = Q K^T on blocks
    P = softmax(L, S, scale, causal)  # block-sparse row softmax
    O = dsd(L, P, v)                  # O = P V
    C = dds(L, a, S)                  # C = A S
    O = attention(L, q, k, v, scale, causal)   # fused SDD -> softmax -> DSD
    dq, dk, dv = attention_backward(L, q, k, v, do, scale, causal)
    O = attention_autograd(L, q, k, v, scale, causal)   # differentiable

Operation semantics follow the three block-sparse modes and the softmax of
Triton issue 117 ("question on blocksparse"); see include/bsattn.h.
"""
from __future__ import annotations

import ctypes as C
import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from . import _lib
from ._lib import (AcsrTerm, BsError, BS_BF16, BS_CAUSAL, BS_F16, BS_F32, BS_F8E4M3, BS_TRANS_A, BS_TRANS_B, check,
                   lib)

__all__ = ["Layout", "sdd", "softmax", "dsd", "dds", "attention", "softmax_backward", "dsd_t",
           "attention_backward", "attention_backward_fused", "attention_autograd", "BsError", "lib"]


def _torch():
    import torch
    return torch


def _stream(device) -> C.c_void_p:
    torch = _torch()
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return BS_F32
    if t.dtype == torch.bfloat16:
        return BS_BF16
    if t.dtype == torch.float16:
        return BS_F16
    if t.dtype == getattr(torch, "float8_e4m3fn", None):
        return BS_F8E4M3
    raise TypeError(f"dense operands must be float32, bfloat16, float16 or float8_e4m3fn, got {t.dtype}")


def _check_dense(name, t, ndim=4):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")


def _ptr(t) -> C.c_void_p:
    return C.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else 0)


class Layout:
    """A built block layout: device block-CSR/CSC tables (owned by the library)."""

    def __init__(self, layout, block: int, device=None, _handle=None):
        torch = _torch()
        if _handle is not None:
            self._h = _handle
        else:
            if not torch.cuda.is_available():
                raise RuntimeError("Layout needs a visible GPU (HIP device)")
            lay = torch.as_tensor(np.asarray(layout) if not isinstance(layout, torch.Tensor) else layout)
            if lay.dim() != 3:
                raise ValueError("layout must be [H, nbr, nbc]")
            dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
            lay = lay.to(device=dev, dtype=torch.uint8).contiguous()
            H, nbr, nbc = lay.shape
            h = C.c_void_p()
            with torch.cuda.device(dev):
                check(lib().bs_layout_build(_ptr(lay), H, nbr, nbc, block, _stream(dev), C.byref(h)))
            self._h = h
        self._read_info()

    @classmethod
    def acsr(cls, terms: Sequence[Tuple[int, int, int, int, int, int]], H: int, nbr: int, nbc: int,
             block: int, device=None) -> "Layout":
        """Layout from affine row terms (row_begin, row_end, slope, offset,
        stride, count), the same for every head."""
        torch = _torch()
        if not torch.cuda.is_available():
            raise RuntimeError("Layout needs a visible GPU (HIP device)")
        arr = (AcsrTerm * max(1, len(terms)))()
        for i, t in enumerate(terms):
            arr[i] = AcsrTerm(*[int(v) for v in t])
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        h = C.c_void_p()
        with torch.cuda.device(dev):
            check(lib().bs_layout_build_acsr(arr, len(terms), H, nbr, nbc, block, _stream(dev), C.byref(h)))
        return cls(None, block, _handle=h)

    def _read_info(self):
        H, nbr, nbc, b = C.c_int(), C.c_int(), C.c_int(), C.c_int()
        nnz = C.c_int64()
        check(lib().bs_layout_info(self._h, C.byref(H), C.byref(nbr), C.byref(nbc), C.byref(b), None))
        check(lib().bs_layout_nnz(self._h, C.byref(nnz)))
        self.H, self.nbr, self.nbc, self.block, self.nnz = H.value, nbr.value, nbc.value, b.value, nnz.value

    def kv_share(self) -> Tuple[int, int]:
        """(rows, stride) of the K/V sharing plan: block rows per workgroup
        of the fused attention and their distance; (1, 0) without a plan."""
        rows, stride = C.c_int(), C.c_int()
        check(lib().bs_layout_kv_share(self.handle, C.byref(rows), C.byref(stride)))
        return rows.value, stride.value

    def set_kv_share(self, enable: Optional[bool]) -> None:
        """Use (True) or skip (False) the sharing plan in the fused
        attention; None (the default) uses it where it measured faster
        (16-bit operands, blocks of 64)."""
        mode = -1 if enable is None else (1 if enable else 0)
        check(lib().bs_layout_set_kv_share(self.handle, mode))

    @property
    def handle(self) -> C.c_void_p:
        if self._h is None:
            raise RuntimeError("layout was freed")
        return self._h

    def export(self) -> Dict[str, np.ndarray]:
        """Copy the tables to host numpy int32 arrays."""
        n = self.nnz
        out = {
            "row_ptr": np.zeros(self.H * self.nbr + 1, np.int32),
            "col_idx": np.zeros(n, np.int32),
            "col_ptr": np.zeros(self.H * self.nbc + 1, np.int32),
            "row_idx": np.zeros(n, np.int32),
            "blk_id": np.zeros(n, np.int32),
        }
        ptrs = [a.ctypes.data_as(C.POINTER(C.c_int32)) for a in out.values()]
        check(lib().bs_layout_export(self.handle, *ptrs))
        return out

    def free(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().bs_layout_free(self._h)
        self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def _empty(shape, dtype, device):
    return _torch().empty(shape, dtype=dtype, device=device)


def _out(out, shape, dtype, device, name="out"):
    """A new output tensor, or the caller's after checking that the kernels
    can write all of it (shape, dtype, device, contiguity)."""
    shape = tuple(shape)
    if out is None:
        return _empty(shape, dtype, device)
    if (tuple(out.shape) != shape or out.dtype != dtype or not out.is_cuda or out.device != device
            or not out.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} on {device}")
    return out


def _trans(trans_a: bool, trans_b: bool) -> int:
    return (BS_TRANS_A if trans_a else 0) | (BS_TRANS_B if trans_b else 0)


def sdd(L: Layout, a, b, out=None, trans_a: bool = False, trans_b: bool = False):
    """S[z, k] = a'[z, h, r-block, :] @ b'[z, h, c-block, :]^T for each stored
    block, where a' = a ([Z, H, nbr*b, K]) or, with trans_a, a is stored as
    [Z, H, K, nbr*b] and a' is its transpose; b' likewise ([Z, H, nbc*b, K],
    or [Z, H, K, nbc*b] with trans_b)."""
    torch = _torch()
    _check_dense("a", a)
    _check_dense("b", b)
    Z, H = a.shape[:2]
    K = a.shape[2] if trans_a else a.shape[3]
    Na, Nb = L.nbr * L.block, L.nbc * L.block
    if a.dtype != b.dtype or tuple(a.shape) != ((Z, H, K, Na) if trans_a else (Z, H, Na, K)) \
            or tuple(b.shape) != ((Z, H, K, Nb) if trans_b else (Z, H, Nb, K)) or H != L.H:
        raise ValueError("a must be [Z, H, nbr*b, K] ([Z, H, K, nbr*b] with trans_a) and b [Z, H, nbc*b, K] "
                         "([Z, H, K, nbc*b] with trans_b), of one dtype")
    out = _out(out, (Z, L.nnz, L.block, L.block), torch.float32, a.device)
    if trans_a or trans_b:
        check(lib().bs_sdd_ex(L.handle, _ptr(a), _ptr(b), _ptr(out), Z, K, _trans(trans_a, trans_b), _dtype_code(a),
                              _stream(a.device)))
    else:
        check(lib().bs_sdd(L.handle, _ptr(a), _ptr(b), _ptr(out), Z, K, _dtype_code(a), _stream(a.device)))
    return out


def _mask_ptrs(L: Layout, Z: int, device, attn_mask, key_padding_mask):
    """Validated pointers of the optional dense additive masks: attn_mask
    float32 [nbr*b, nbc*b] (shared by batch and heads), key_padding_mask
    float32 [Z, nbc*b]; None for an absent mask."""
    torch = _torch()
    ptrs = []
    for name, m, shape in (("attn_mask", attn_mask, (L.nbr * L.block, L.nbc * L.block)),
                           ("key_padding_mask", key_padding_mask, (Z, L.nbc * L.block))):
        if m is None:
            ptrs.append(None)
            continue
        _check_dense(name, m, ndim=2)
        if m.dtype != torch.float32 or tuple(m.shape) != shape:
            raise ValueError(f"{name} must be float32 {list(shape)}")
        if m.device != device:
            raise ValueError(f"{name} must be on {device}")
        ptrs.append(_ptr(m))
    return ptrs


def softmax(L: Layout, s, scale: float, causal: bool = False, out=None, inplace: bool = False, attn_mask=None,
            key_padding_mask=None):
    """Block-sparse row softmax of SDD output: scale, plus the optional dense
    additive masks (attn_mask [nbr*b, nbc*b], key_padding_mask [Z, nbc*b],
    float32, -inf hides), then the causal mask."""
    torch = _torch()
    _check_dense("s", s)
    if s.dtype != torch.float32 or s.shape[1:] != (L.nnz, L.block, L.block):
        raise ValueError("s must be float32 [Z, nnz, b, b]")
    am, kp = _mask_ptrs(L, s.shape[0], s.device, attn_mask, key_padding_mask)
    out = s if inplace else _out(out, s.shape, torch.float32, s.device)
    flags = BS_CAUSAL if causal else 0
    if am is None and kp is None:
        check(lib().bs_softmax(L.handle, _ptr(s), _ptr(out), s.shape[0], float(scale), flags, _stream(s.device)))
    else:
        check(lib().bs_softmax_masked(L.handle, _ptr(s), _ptr(out), s.shape[0], float(scale), flags, am, kp,
                                      _stream(s.device)))
    return out


def dsd(L: Layout, p, b, out=None, trans_a: bool = False, trans_b: bool = False):
    """C[z, h, r-block, :] = sum over stored (h, r, c) of p[z, k] @ b[z, h, c-block, :].
    trans_a: the block matrix transposed (C[z, h, c-block, :] = sum of
    p[z, k]^T @ b[z, h, r-block, :], as dsd_t); trans_b: b stored as
    [Z, H, Nd, rows] and used transposed."""
    torch = _torch()
    _check_dense("p", p)
    _check_dense("b", b)
    Z, H = b.shape[:2]
    Nd = b.shape[2] if trans_b else b.shape[3]
    n_in = (L.nbr if trans_a else L.nbc) * L.block
    n_out = (L.nbc if trans_a else L.nbr) * L.block
    if p.dtype != torch.float32 or p.shape != (Z, L.nnz, L.block, L.block):
        raise ValueError("p must be float32 [Z, nnz, b, b]")
    if H != L.H or tuple(b.shape) != ((Z, H, Nd, n_in) if trans_b else (Z, H, n_in, Nd)):
        raise ValueError(f"b must be [Z, H, {n_in}, Nd] ([Z, H, Nd, {n_in}] with trans_b)")
    out = _out(out, (Z, H, n_out, Nd), b.dtype, b.device)
    if trans_a or trans_b:
        check(lib().bs_dsd_ex(L.handle, _ptr(p), _ptr(b), _ptr(out), Z, Nd, _trans(trans_a, trans_b),
                              _dtype_code(b), _stream(b.device)))
    else:
        check(lib().bs_dsd(L.handle, _ptr(p), _ptr(b), _ptr(out), Z, Nd, _dtype_code(b), _stream(b.device)))
    return out


def dds(L: Layout, a, s, out=None, trans_a: bool = False, trans_b: bool = False):
    """C[z, h, :, c-block] = sum over stored (h, r, c) of a[z, h, :, r-block] @ s[z, k].
    trans_a: a stored as [Z, H, rows, M] and used transposed; trans_b: the
    block matrix transposed (C[z, h, :, r-block] = sum of
    a[z, h, :, c-block] @ s[z, k]^T)."""
    torch = _torch()
    _check_dense("a", a)
    _check_dense("s", s)
    Z, H = a.shape[:2]
    M = a.shape[3] if trans_a else a.shape[2]
    n_in = (L.nbc if trans_b else L.nbr) * L.block
    n_out = (L.nbr if trans_b else L.nbc) * L.block
    if s.dtype != torch.float32 or s.shape != (Z, L.nnz, L.block, L.block):
        raise ValueError("s must be float32 [Z, nnz, b, b]")
    if H != L.H or tuple(a.shape) != ((Z, H, n_in, M) if trans_a else (Z, H, M, n_in)):
        raise ValueError(f"a must be [Z, H, M, {n_in}] ([Z, H, {n_in}, M] with trans_a)")
    out = _out(out, (Z, H, M, n_out), a.dtype, a.device)
    if trans_a or trans_b:
        check(lib().bs_dds_ex(L.handle, _ptr(a), _ptr(s), _ptr(out), Z, M, _trans(trans_a, trans_b),
                              _dtype_code(a), _stream(a.device)))
    else:
        check(lib().bs_dds(L.handle, _ptr(a), _ptr(s), _ptr(out), Z, M, _dtype_code(a), _stream(a.device)))
    return out


def attention(L: Layout, q, k, v, scale: Optional[float] = None, causal: bool = False, out=None, attn_mask=None,
              key_padding_mask=None, return_lse: bool = False, lse=None):
    """Fused block-sparse attention O = softmax(scale q k^T + mask) v; the
    mask is the layout's, the optional dense additive masks (see softmax)
    and the causal one. With return_lse, also the float32 [Z, H, Nq] row
    log-sum-exp of the masked scaled scores (-inf for empty rows), written
    by the same kernel: returns (out, lse).
    fp8: q and k of dtype torch.float8_e4m3fn (the score product on the fp8
    matrix cores), v bfloat16; out is bfloat16 (d = 128, blocks >= 32)."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_dense(n, t)
    Z, H, Nq, d = q.shape
    fp8 = q.dtype == getattr(torch, "float8_e4m3fn", None)
    if fp8:
        if k.dtype != q.dtype or v.dtype != torch.bfloat16:
            raise ValueError("fp8 attention takes q, k as float8_e4m3fn and v as bfloat16")
    elif not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    if (H, Nq) != (L.H, L.nbr * L.block) or k.shape != (Z, H, L.nbc * L.block, d) or v.shape != k.shape:
        raise ValueError("q must be [Z, H, nbr*b, d]; k, v [Z, H, nbc*b, d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    am, kp = _mask_ptrs(L, Z, q.device, attn_mask, key_padding_mask)
    out = _out(out, q.shape, v.dtype, q.device)
    flags = BS_CAUSAL if causal else 0
    if return_lse:
        lse = _out(lse, (Z, H, Nq), _torch().float32, q.device, "lse")
        check(lib().bs_attention_fwd(L.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), Z, d, float(scale),
                                     flags, am, kp, _dtype_code(q), _stream(q.device)))
        return out, lse
    if am is None and kp is None:
        check(lib().bs_attention(L.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), Z, d, float(scale), flags,
                                 _dtype_code(q), _stream(q.device)))
    else:
        check(lib().bs_attention_masked(L.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), Z, d, float(scale), flags,
                                        am, kp, _dtype_code(q), _stream(q.device)))
    return out


# ------------------------------------------------------------------ backward

def softmax_backward(L: Layout, p, dp, scale: float, out=None, inplace: bool = False):
    """Gradient of softmax with respect to its input: for each query row,
    dS = scale * p * (dp - sum over the row of p * dp)."""
    torch = _torch()
    _check_dense("p", p)
    _check_dense("dp", dp)
    if p.dtype != torch.float32 or p.shape[1:] != (L.nnz, L.block, L.block) or dp.shape != p.shape \
            or dp.dtype != torch.float32:
        raise ValueError("p and dp must be float32 [Z, nnz, b, b]")
    out = dp if inplace else _out(out, p.shape, torch.float32, p.device)
    check(lib().bs_softmax_backward(L.handle, _ptr(p), _ptr(dp), _ptr(out), p.shape[0], float(scale),
                                    _stream(p.device)))
    return out


def dsd_t(L: Layout, s, b, out=None):
    """C[z, h, c-block, :] = sum over stored (h, r, c) of s[z, k]^T @ b[z, h, r-block, :]."""
    torch = _torch()
    _check_dense("s", s)
    _check_dense("b", b)
    Z, H, Nb, Nd = b.shape
    if s.dtype != torch.float32 or s.shape != (Z, L.nnz, L.block, L.block):
        raise ValueError("s must be float32 [Z, nnz, b, b]")
    if (H, Nb) != (L.H, L.nbr * L.block):
        raise ValueError("b must be [Z, H, nbr*b, Nd]")
    out = _out(out, (Z, H, L.nbc * L.block, Nd), b.dtype, b.device)
    check(lib().bs_dsd_t(L.handle, _ptr(s), _ptr(b), _ptr(out), Z, Nd, _dtype_code(b), _stream(b.device)))
    return out


def attention_backward(L: Layout, q, k, v, do, scale: Optional[float] = None, causal: bool = False,
                       workspace: Optional[Tuple] = None, attn_mask=None, key_padding_mask=None):
    """(dq, dk, dv) of attention() for the output gradient do, in one library
    call: P recomputed by SDD and softmax (under the same dense masks),
    dP = SDD(do, v), dS = softmax gradient, dq = DSD(dS, k),
    dk = DSD^T(dS, q), dv = DSD^T(P, do).
    workspace: optional pair of float32 [Z, nnz, b, b] tensors."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        _check_dense(n, t)
    Z, H, Nq, d = q.shape
    if not (q.dtype == k.dtype == v.dtype == do.dtype):
        raise ValueError("q, k, v, do must share a dtype")
    if (H, Nq) != (L.H, L.nbr * L.block) or k.shape != (Z, H, L.nbc * L.block, d) or v.shape != k.shape \
            or do.shape != q.shape:
        raise ValueError("q and do must be [Z, H, nbr*b, d]; k, v [Z, H, nbc*b, d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ws_shape = (Z, L.nnz, L.block, L.block)
    ws_s, ws_p = workspace if workspace is not None else (None, None)
    ws_s = _out(ws_s, ws_shape, torch.float32, q.device, "workspace")
    ws_p = _out(ws_p, ws_shape, torch.float32, q.device, "workspace")
    am, kp = _mask_ptrs(L, Z, q.device, attn_mask, key_padding_mask)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    flags = BS_CAUSAL if causal else 0
    if am is None and kp is None:
        check(lib().bs_attention_backward(L.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq), _ptr(dk),
                                          _ptr(dv), _ptr(ws_s), _ptr(ws_p), Z, d, float(scale), flags,
                                          _dtype_code(q), _stream(q.device)))
    else:
        check(lib().bs_attention_backward_masked(L.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(dq),
                                                 _ptr(dk), _ptr(dv), _ptr(ws_s), _ptr(ws_p), Z, d, float(scale),
                                                 flags, am, kp, _dtype_code(q), _stream(q.device)))
    return dq, dk, dv


def attention_backward_fused(L: Layout, q, k, v, o, lse, do, scale: Optional[float] = None, causal: bool = False,
                             attn_mask=None, key_padding_mask=None, workspace=None, out=None, noalloc: bool = False):
    """(dq, dk, dv) of attention() from its inputs, its output o and row
    log-sum-exp lse (attention(..., return_lse=True)) and the output
    gradient do, on the fused backward kernels (S and P never reach
    memory). Same scale, causal flag and masks as the forward.
    workspace: optional float32 [Z, H, Nq] tensor, scratch for the rows'
    D = rowsum(do * o) terms (its contents afterwards are unspecified).
    out: optional (dq, dk, dv) tensors to write.
    noalloc: call bs_attention_bwd_noalloc, which keeps D in the library's
    static device buffer (at most 2^21 query rows) and allocates nothing;
    with `out` given this call allocates no device memory at all."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_dense(n, t)
    _check_dense("lse", lse, ndim=3)
    Z, H, Nq, d = q.shape
    if not (q.dtype == k.dtype == v.dtype == o.dtype == do.dtype):
        raise ValueError("q, k, v, o, do must share a dtype")
    if (H, Nq) != (L.H, L.nbr * L.block) or k.shape != (Z, H, L.nbc * L.block, d) or v.shape != k.shape \
            or o.shape != q.shape or do.shape != q.shape:
        raise ValueError("q, o, do must be [Z, H, nbr*b, d]; k, v [Z, H, nbc*b, d]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (Z, H, Nq):
        raise ValueError("lse must be float32 [Z, H, nbr*b]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    am, kp = _mask_ptrs(L, Z, q.device, attn_mask, key_padding_mask)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = (_out(t, like.shape, like.dtype, like.device, n)
                      for t, like, n in zip(out, (q, k, v), ("dq", "dk", "dv")))
    flags = BS_CAUSAL if causal else 0
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace (D lives in the library's static buffer)")
        check(lib().bs_attention_bwd_noalloc(L.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                             _ptr(dq), _ptr(dk), _ptr(dv), Z, d, float(scale), flags, am, kp,
                                             _dtype_code(q), _stream(q.device)))
        return dq, dk, dv
    ws = _out(workspace, (Z, H, Nq), torch.float32, q.device, "workspace")
    check(lib().bs_attention_bwd(L.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                                 _ptr(dk), _ptr(dv), _ptr(ws), Z, d, float(scale), flags, am, kp,
                                 _dtype_code(q), _stream(q.device)))
    return dq, dk, dv


_AUTOGRAD_FN = None


def _autograd_fn():
    """The torch.autograd.Function pairing attention() with
    attention_backward() (built on first use, so importing this package
    does not import torch)."""
    global _AUTOGRAD_FN
    if _AUTOGRAD_FN is None:
        torch = _torch()

        class BlockSparseAttention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, L, scale, causal, attn_mask, key_padding_mask):
                o, lse = attention(L, q, k, v, scale, causal, attn_mask=attn_mask,
                                   key_padding_mask=key_padding_mask, return_lse=True)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.L, ctx.scale, ctx.causal = L, scale, causal
                ctx.masks = (attn_mask, key_padding_mask)
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                am, kp = ctx.masks
                dq, dk, dv = attention_backward_fused(ctx.L, q, k, v, o, lse, do.contiguous(), ctx.scale,
                                                      ctx.causal, attn_mask=am, key_padding_mask=kp)
                return dq, dk, dv, None, None, None, None, None

        _AUTOGRAD_FN = BlockSparseAttention
    return _AUTOGRAD_FN


def attention_autograd(L: Layout, q, k, v, scale: Optional[float] = None, causal: bool = False, attn_mask=None,
                       key_padding_mask=None):
    """attention() as a differentiable torch op (forward: the fused kernel,
    which also writes the row log-sum-exp; backward: the fused backward
    kernels). The dense masks are constants (no gradient)."""
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _autograd_fn().apply(q, k, v, L, float(scale), bool(causal), attn_mask, key_padding_mask)

