// Row-block kernel instantiations: the fused attention (fp32, and the 16-bit
// types where the 32-rows-per-wave kernel does not apply), the SDD and DSD
// for contraction / output widths of 64 and 128, and the DSD of the
// transposed block matrix (attention backward). The kernel itself, with its
// description, is in rowblock.h.
#include "rowblock.h"

namespace bsa {

int launch_attention(const bs_layout* L, const AttnArgs& at, hipStream_t s) {
  if (at.dt != BS_F32) {
    const int rc = launch_attention_wide(L, at, s);
    if (rc != kNotApplicable) return rc;
    if (at.dt == BS_F8E4M3) return fail(BS_ERR_UNSUPPORTED, "BS_F8E4M3 attention: no kernel for this shape");
  }
  if (at.am != nullptr || at.kp != nullptr) return launch_attention_masked(L, at, s);
  const int rc = launch_attention_band(L, at, s);
  if (rc != kNotApplicable) return rc;
  Args a{at.Q, at.K, at.V, at.O, nullptr, at.Z, at.scale * kLog2e, at.causal};
  a.use_band = L->band_off != nullptr;
  a.lse = at.lse;
  return run_mode<MODE_ATTN>(L, a, at.d, at.dt, s);
}

int launch_sdd_rowblock(const bs_layout* L, const void* A, const void* B, float* S, int Z, int K, bs_dtype dt,
                        hipStream_t s) {
  if (K != 64 && K != 128) return kNotApplicable;
  const Args a{A, B, nullptr, nullptr, S, Z, 1.f, false};
  return run_mode<MODE_SDD>(L, a, K, dt, s);
}

int launch_dsd_rowblock(const bs_layout* L, const float* P, const void* B, void* C, int Z, int Nd, bs_dtype dt,
                        hipStream_t s) {
  if (Nd != 64 && Nd != 128) return kNotApplicable;
  const Args a{nullptr, nullptr, B, C, const_cast<float*>(P), Z, 1.f, false};
  return run_mode<MODE_DSD>(L, a, Nd, dt, s);
}

int launch_dsd_t(const bs_layout* L, const float* S, const void* B, void* C, int Z, int Nd, bs_dtype dt,
                 hipStream_t s) {
  if (Nd != 64 && Nd != 128) return fail(BS_ERR_UNSUPPORTED, "bs_dsd_t supports Nd = 64 or 128");
  const Args a{nullptr, nullptr, B, C, const_cast<float*>(S), Z, 1.f, false};
  return run_mode<MODE_DSDT>(L, a, Nd, dt, s);
}

}  // namespace bsa
