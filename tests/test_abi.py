"""The C-ABI library: it loads, exports every function include/bsattn.h
declares, and rejects invalid arguments before any HIP call (so these run on a
CPU-only host). No compute call is made here."""
import ctypes as C
import os
import re

import pytest

from block_sparse_matmul_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsattn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bs_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("bs_layout_build", "bs_layout_build_acsr", "bs_layout_nnz", "bs_sdd", "bs_softmax", "bs_dsd", "bs_dds",
              "bs_attention", "bs_last_error", "bs_layout_free", "bs_layout_export",
              "bs_softmax_backward", "bs_dsd_t", "bs_attention_backward", "bs_layout_kv_share",
              "bs_layout_set_kv_share"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for n in _declared_functions():
        assert hasattr(L, n), n
    assert set(_declared_functions()) == set(_lib.SIGNATURES), "binding signatures out of date"
    assert L.bs_version() >= 100


def test_header_constants_match_binding():
    """The dtype, flag and error codes the binding passes are the header's."""
    src = open(HEADER).read()
    vals = {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(BS_[A-Z0-9_]+)\s*=\s*(-?\d+)", src)}
    for name in ("BS_F32", "BS_BF16", "BS_F16", "BS_F8E4M3", "BS_CAUSAL", "BS_TRANS_A", "BS_TRANS_B", "BS_OK", "BS_ERR_INVALID_ARG", "BS_ERR_UNSUPPORTED",
                 "BS_ERR_SHAPE", "BS_ERR_HIP", "BS_ERR_OOM", "BS_ERR_NO_DEVICE"):
        assert vals[name] == getattr(_lib, name), name


def _build(layout_ptr, H, nbr, nbc, block):
    h = C.c_void_p()
    rc = _lib.lib().bs_layout_build(layout_ptr, H, nbr, nbc, block, None, C.byref(h))
    return rc, h


@pytest.mark.parametrize("block", [0, 8, 17, 48, 256])
def test_unsupported_block_rejected_first(block):
    buf = (C.c_uint8 * 4)()
    rc, h = _build(C.cast(buf, C.c_void_p), 1, 2, 2, block)
    assert rc == _lib.BS_ERR_UNSUPPORTED and not h.value
    assert b"block" in _lib.lib().bs_last_error()


def test_bad_sizes_and_null_pointers():
    buf = (C.c_uint8 * 4)()
    assert _build(C.cast(buf, C.c_void_p), 0, 2, 2, 16)[0] == _lib.BS_ERR_INVALID_ARG
    assert _build(C.cast(buf, C.c_void_p), 1, -1, 2, 16)[0] == _lib.BS_ERR_INVALID_ARG
    assert _build(None, 1, 2, 2, 16)[0] == _lib.BS_ERR_INVALID_ARG
    assert _build(C.cast(buf, C.c_void_p), 4096, 4096, 4096, 16)[0] == _lib.BS_ERR_SHAPE
    assert _lib.lib().bs_layout_build(C.cast(buf, C.c_void_p), 1, 2, 2, 16, None, None) == _lib.BS_ERR_INVALID_ARG


def test_acsr_term_validation():
    L = _lib.lib()
    h = C.c_void_p()
    bad = (_lib.AcsrTerm * 1)(_lib.AcsrTerm(5, 2, 1, 0, 1, 1))
    assert L.bs_layout_build_acsr(bad, 1, 1, 8, 8, 16, None, C.byref(h)) == _lib.BS_ERR_INVALID_ARG
    neg = (_lib.AcsrTerm * 1)(_lib.AcsrTerm(0, 2, 1, 0, 1, -3))
    assert L.bs_layout_build_acsr(neg, 1, 1, 8, 8, 16, None, C.byref(h)) == _lib.BS_ERR_INVALID_ARG
    assert L.bs_layout_build_acsr(None, 2, 1, 8, 8, 16, None, C.byref(h)) == _lib.BS_ERR_INVALID_ARG
    assert L.bs_layout_build_acsr(bad, 1, 1, 8, 8, 24, None, C.byref(h)) == _lib.BS_ERR_UNSUPPORTED


def test_compute_calls_reject_null_handle():
    L = _lib.lib()
    assert L.bs_sdd(None, None, None, None, 1, 64, 0, None) == _lib.BS_ERR_INVALID_ARG
    assert L.bs_softmax(None, None, None, 1, 1.0, 0, None) == _lib.BS_ERR_INVALID_ARG
    assert L.bs_dsd(None, None, None, None, 1, 64, 0, None) == _lib.BS_ERR_INVALID_ARG
    assert L.bs_dds(None, None, None, None, 1, 64, 0, None) == _lib.BS_ERR_INVALID_ARG
    assert L.bs_attention(None, None, None, None, None, 1, 64, 1.0, 0, 0, None) == _lib.BS_ERR_INVALID_ARG
    assert L.bs_softmax_backward(None, None, None, None, 1, 1.0, None) == _lib.BS_ERR_INVALID_ARG
    assert L.bs_dsd_t(None, None, None, None, 1, 64, 0, None) == _lib.BS_ERR_INVALID_ARG
    assert L.bs_attention_backward(None, None, None, None, None, None, None, None, None, None, 1, 64, 1.0, 0, 0,
                                   None) == _lib.BS_ERR_INVALID_ARG
    assert L.bs_layout_info(None, None, None, None, None, None) == _lib.BS_ERR_INVALID_ARG
    n = C.c_int64(-1)
    assert L.bs_layout_nnz(None, C.byref(n)) == _lib.BS_ERR_INVALID_ARG and n.value == -1
    assert L.bs_layout_export(None, None, None, None, None, None) == _lib.BS_ERR_INVALID_ARG
    rows, stride = C.c_int(-1), C.c_int(-1)
    assert L.bs_layout_kv_share(None, C.byref(rows), C.byref(stride)) == _lib.BS_ERR_INVALID_ARG
    assert rows.value == -1 and stride.value == -1
    assert L.bs_layout_set_kv_share(None, 1) == _lib.BS_ERR_INVALID_ARG
    L.bs_layout_free(None)  # ignored


def test_no_device_reported_on_cpu_host():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    buf = (C.c_uint8 * 4)(1, 0, 0, 1)
    rc, h = _build(C.cast(buf, C.c_void_p), 1, 2, 2, 16)
    assert rc == _lib.BS_ERR_NO_DEVICE and not h.value
