// Fused block-sparse attention with the dense additive masks (Triton issue
// 117, "question on blocksparse": dense masks may be passed alongside the
// layout): the row-block kernel's MODE_ATTN_MASKED instantiation. After the
// score product each lane adds log2(e) * (attn_mask[query][key] +
// kp_mask[z][key]) to its scores (16-byte reads of 4 consecutive keys), then
// the causal mask and the streaming softmax run as without masks. The
// 32-rows-per-wave 16-bit kernel paces its LDS transfers by counting the
// vector-memory operations in flight, which extra mask loads would upset,
// so every type takes the row-block kernel here.
#include "rowblock.h"

namespace bsa {

int launch_attention_masked(const bs_layout* L, const void* Q, const void* K, const void* V, void* O, int Z, int d,
                            float scale, bool causal, const float* am, const float* kp, bs_dtype dt, hipStream_t s) {
  Args a{Q, K, V, O, nullptr, Z, scale * kLog2e, causal};
  a.use_band = L->band_off != nullptr;
  a.am = am;
  a.kp = kp;
  return run_mode<MODE_ATTN_MASKED>(L, a, d, dt, s);
}

}  // namespace bsa
