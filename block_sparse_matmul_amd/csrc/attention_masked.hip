// Fused block-sparse attention with the dense additive masks (Triton issue
// 117, "question on blocksparse": dense masks may be passed alongside the
// layout): the row-block kernel's MODE_ATTN_MASKED instantiation. After the
// score product each lane adds log2(e) * (attn_mask[query][key] +
// kp_mask[z][key]) to its scores (16-byte reads of 4 consecutive keys), then
// the causal mask and the streaming softmax run as without masks. The 16-bit
// types with blocks of 32 to 128 take the 32-rows-per-wave kernel's masked
// variant instead.
#include "rowblock.h"

namespace bsa {

int launch_attention_masked(const bs_layout* L, const AttnArgs& at, hipStream_t s) {
  Args a{at.Q, at.K, at.V, at.O, nullptr, at.Z, at.scale * kLog2e, at.causal};
  a.use_band = L->band_off != nullptr;
  a.am = at.am;
  a.kp = at.kp;
  a.lse = at.lse;
  return run_mode<MODE_ATTN_MASKED>(L, a, at.d, at.dt, s);
}

}  // namespace bsa
