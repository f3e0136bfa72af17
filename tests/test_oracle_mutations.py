"""Planted mistakes in the oracle must make its pins fail.

Each case changes one expression of the oracle's source (in a child process,
on the CPU) to a plausible slip -- a transposed operand, a dropped scale, a
flipped or off-by-one mask, a wrong block index, a NaN on empty rows, a
dropped term of the softmax gradient -- and
runs the oracle pin suite against it. A pin suite that still passes would not
be able to tell that mistake from the method.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "sdd_block_transposed": (
        "S[z, k] = A[z, h, r * b:(r + 1) * b, :] @ B[z, h, c * b:(c + 1) * b, :].T",
        "S[z, k] = (A[z, h, r * b:(r + 1) * b, :] @ B[z, h, c * b:(c + 1) * b, :].T).T"),
    "softmax_scale_dropped": (
        "x = np.concatenate([scale * S[z, k] for k in ks], axis=1)",
        "x = np.concatenate([S[z, k] for k in ks], axis=1)"),
    "causal_diagonal_hidden": (
        "x = np.where(kj <= qi, x, -np.inf)",
        "x = np.where(kj < qi, x, -np.inf)"),
    "element_mask_causal_flipped": (
        "m = m & (np.arange(nk)[None, None, :] <= np.arange(nq)[None, :, None])",
        "m = m & (np.arange(nk)[None, None, :] >= np.arange(nq)[None, :, None])"),
    "softmax_nan_on_empty_rows": (
        "            p = np.divide(e, s, out=np.zeros_like(e), where=s > 0)\n            for n, k in enumerate(ks):",
        "            p = e / s\n            for n, k in enumerate(ks):"),
    "dsd_p_transposed": (
        "C[z, h, r * b:(r + 1) * b, :] += P[z, k] @ B[z, h, c * b:(c + 1) * b, :]",
        "C[z, h, r * b:(r + 1) * b, :] += P[z, k].T @ B[z, h, c * b:(c + 1) * b, :]"),
    "dsd_wrong_value_block": (
        "C[z, h, r * b:(r + 1) * b, :] += P[z, k] @ B[z, h, c * b:(c + 1) * b, :]",
        "C[z, h, r * b:(r + 1) * b, :] += P[z, k] @ B[z, h, r * b:(r + 1) * b, :]"),
    "dds_s_transposed": (
        "C[z, h, :, c * b:(c + 1) * b] += A[z, h, :, r * b:(r + 1) * b] @ S[z, k]",
        "C[z, h, :, c * b:(c + 1) * b] += A[z, h, :, r * b:(r + 1) * b] @ S[z, k].T"),
    "dense_attention_scale_dropped": (
        "x = scale * (Q[z, h] @ K[z, h].T)",
        "x = (Q[z, h] @ K[z, h].T)"),
    "lut_row_ptr_shifted": (
        "row_ptr[1:] = np.cumsum(row_counts)",
        "row_ptr[:-1] = np.cumsum(row_counts)"),
    "lut_csc_blk_id_swapped": (
        '"blk_id": ids[th, tr, tc].astype(np.int32)',
        '"blk_id": ids[th, tc % nbr, tr % nbc].astype(np.int32)'),
    "acsr_stride_ignored": (
        "c = slope * r + offset + stride * k",
        "c = slope * r + offset + k"),
    "softmax_backward_row_term_dropped": (
        "dS[z, k] = scale * P[z, k] * (dP[z, k] - D)",
        "dS[z, k] = scale * P[z, k] * dP[z, k]"),
    "softmax_backward_scale_dropped": (
        "dS[z, k] = scale * P[z, k] * (dP[z, k] - D)",
        "dS[z, k] = P[z, k] * (dP[z, k] - D)"),
    "dsd_t_block_not_transposed": (
        "C[z, h, c * b:(c + 1) * b, :] += S[z, k].T @ B[z, h, r * b:(r + 1) * b, :]",
        "C[z, h, c * b:(c + 1) * b, :] += S[z, k] @ B[z, h, r * b:(r + 1) * b, :]"),
    "dense_backward_dk_untransposed": (
        "dK[z, h] = scale * (dX.T @ Q[z, h])",
        "dK[z, h] = scale * (dX @ Q[z, h])"),
    "dense_backward_dv_untransposed": (
        "dV[z, h] = P.T @ dO[z, h]",
        "dV[z, h] = P @ dO[z, h]"),
    "mask_attn_transposed": (
        "out = out + attn_mask[np.ix_(qi, kj)]",
        "out = out + attn_mask[np.ix_(kj, qi)].T"),
    "mask_key_padding_on_queries": (
        "out = out + kp_mask[z, kj][None, :]",
        "out = out + kp_mask[z, qi][:, None]"),
    "mask_key_padding_wrong_batch": (
        "out = out + kp_mask[z, kj][None, :]",
        "out = out + kp_mask[0, kj][None, :]"),
    "softmax_dense_mask_dropped": (
        "x = x + _bias(am, kpm, z, qrows, kcols)",
        "x = x"),
    "dense_backward_mask_dropped": (
        "x = scale * (Q[z, h] @ K[z, h].T) + _bias(am, kpm, z, qall, kall)",
        "x = scale * (Q[z, h] @ K[z, h].T)"),
    "lse_max_term_dropped": (
        "out[z, h] = np.where(ok, mm + np.log(np.where(ok, tot, 1.0)), -np.inf)",
        "out[z, h] = np.where(ok, np.log(np.where(ok, tot, 1.0)), -np.inf)"),
    "dds_t_block_not_transposed": (
        "C[z, h, :, r * b:(r + 1) * b] += A[z, h, :, c * b:(c + 1) * b] @ S[z, k].T",
        "C[z, h, :, r * b:(r + 1) * b] += A[z, h, :, c * b:(c + 1) * b] @ S[z, k]"),
    "rows_wrong_head_mask": (
        "mask = np.repeat(lay[h, r].astype(bool), b)[None, :].repeat(b, axis=0)",
        "mask = np.repeat(lay[0, r].astype(bool), b)[None, :].repeat(b, axis=0)"),
}


def _run_pins(mutant):
    env = dict(os.environ)
    env["BSA_ORACLE_MUTANT"] = json.dumps(list(mutant))
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_lut.py"),
           os.path.join(ROOT, "tests", "test_oracle_ops.py"),
           os.path.join(ROOT, "tests", "test_oracle_backward.py"),
           os.path.join(ROOT, "tests", "test_oracle_masks.py")]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_unmutated_source_passes_through_the_mutation_hook():
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    for name, (old, _) in MUTANTS.items():
        assert src.count(old) >= 1, name
    res = _run_pins(("ALLOWED_BLOCKS = (16, 32, 64, 128)", "ALLOWED_BLOCKS = (16, 32, 64, 128)"))
    assert res.returncode == 0, res.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    res = _run_pins(MUTANTS[name])
    assert res.returncode != 0, f"pins did not catch {name}:\n{res.stdout[-1500:]}"
