// SDD: sampled dense-dense product (Triton issue 117, "question on
// blocksparse": sparse = dense x dense, the first of the three modes).
// For every stored block k = (h, r, c):
//   S[z, k] = A[z, h, r-block, :] . B[z, h, c-block, :]^T      (fp32 out)
//
// Either dense operand may be stored transposed (BS_TRANS_A: A as
// [Z][H][K][nbr*b]; BS_TRANS_B: B as [Z][H][K][nbc*b]); those take the
// generic kernel below with gathered fragments.
//
// K = 64 or 128 runs on the fused attention's row-block kernel (B blocks
// staged through LDS, scores stored from the score registers). Other K take
// the kernel below: one workgroup (4 waves) per (batch, block row), block
// rows taken longest first. The row's output tiles (T x T, T = min(block, 32)) are dealt to the
// waves; each tile is one MFMA accumulation over K with both operands read
// as 16-byte row vectors (A rows are query rows, B rows are key rows), and
// the tile is stored row by row (T consecutive floats per row).
#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

// TA / TB: A stored [Z][H][K][nbr*b] / B stored [Z][H][K][nbc*b] (the
// operand transposed in memory): its fragments are gathered with the row
// length as stride, consecutive lanes reading consecutive addresses.
template <typename E, int BLK, int T, bool TA, bool TB>
__global__ __launch_bounds__(256) void k_sdd(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                                             const int32_t* __restrict__ row_order,
                                             const typename Elem<E>::storage* __restrict__ A,
                                             const typename Elem<E>::storage* __restrict__ B, float* __restrict__ S,
                                             int Z, int H, int nbr, int nbc, int K, int64_t nnz) {
  using St = typename Elem<E>::storage;
  using AccT = typename Acc<T>::type;
  constexpr int G = 64 / T, VEC = Elem<E>::VEC, KC = G * VEC, TPB = BLK / T, NR = T * T / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane % T, g = lane / T;
  // 1-D grid, batch fastest: dispatch follows the longest-first order
  // across the whole batch
  const int hr = row_order[blockIdx.x / Z];
  const int z = blockIdx.x % Z;
  const int h = hr / nbr, r = hr % nbr;
  const int k0 = row_ptr[hr], k1 = row_ptr[hr + 1];
  const int items = (k1 - k0) * TPB * TPB;
  const int64_t zh = (int64_t)z * H + h;
  const int64_t NaT = (int64_t)nbr * BLK, NbT = (int64_t)nbc * BLK;
  for (int it = wave; it < items; it += 4) {
    const int kk = k0 + it / (TPB * TPB);
    const int t = it % (TPB * TPB);
    const int ti = t / TPB, tj = t % TPB;
    const int c = col_idx[kk];
    const int64_t ia = (int64_t)r * BLK + ti * T + li;  // this lane's row of A
    const int64_t jb = (int64_t)c * BLK + tj * T + li;  // and of B
    const St* pa = TA ? A + zh * NaT * K + ia + (int64_t)g * VEC * NaT : A + (zh * NaT + ia) * K + g * VEC;
    const St* pb = TB ? B + zh * NbT * K + jb + (int64_t)g * VEC * NbT : B + (zh * NbT + jb) * K + g * VEC;
    AccT acc = {};
    for (int k = 0; k < K; k += KC) {
      Frag<E> fa, fb;
      if (k + g * VEC < K) {
        if constexpr (TA) fa.load_strided(pa + (int64_t)k * NaT, NaT);
        else fa.load(pa + k);
        if constexpr (TB) fb.load_strided(pb + (int64_t)k * NbT, NbT);
        else fb.load(pb + k);
      } else {
        fa.zero();
        fb.zero();
      }
      mma_frag<T>(acc, fa, fb);
    }
    float* ps = S + ((int64_t)z * nnz + kk) * (BLK * BLK) + (ti * T) * BLK + tj * T + li;
#pragma unroll
    for (int q = 0; q < NR; ++q) ps[acc_row<T>(q, g) * BLK] = acc[q];
  }
}

template <typename E, int BLK, bool TA, bool TB>
int run(const bs_layout* L, const void* A, const void* B, float* S, int Z, int K, hipStream_t s) {
  using St = typename Elem<E>::storage;
  constexpr int T = BLK >= 32 ? 32 : 16;
  hipLaunchKernelGGL((k_sdd<E, BLK, T, TA, TB>), dim3(L->H * L->nbr * Z), dim3(256), 0, s, L->row_ptr, L->col_idx,
                     L->row_order, (const St*)A, (const St*)B, S, Z, L->H, L->nbr, L->nbc, K, L->nnz);
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

template <typename E, bool TA, bool TB>
int run_e(const bs_layout* L, const void* A, const void* B, float* S, int Z, int K, hipStream_t s) {
  switch (L->block) {
    case 16: return run<E, 16, TA, TB>(L, A, B, S, Z, K, s);
    case 32: return run<E, 32, TA, TB>(L, A, B, S, Z, K, s);
    case 64: return run<E, 64, TA, TB>(L, A, B, S, Z, K, s);
    case 128: return run<E, 128, TA, TB>(L, A, B, S, Z, K, s);
  }
  return fail(BS_ERR_UNSUPPORTED, "block must be 16, 32, 64 or 128");
}

template <typename E>
int run_t(const bs_layout* L, const void* A, const void* B, float* S, int Z, int K, int trans, hipStream_t s) {
  switch (trans & (BS_TRANS_A | BS_TRANS_B)) {
    case 0: return run_e<E, false, false>(L, A, B, S, Z, K, s);
    case BS_TRANS_A: return run_e<E, true, false>(L, A, B, S, Z, K, s);
    case BS_TRANS_B: return run_e<E, false, true>(L, A, B, S, Z, K, s);
  }
  return run_e<E, true, true>(L, A, B, S, Z, K, s);
}

}  // namespace

int launch_sdd(const bs_layout* L, const void* A, const void* B, float* S, int Z, int K, int trans, bs_dtype dt,
               hipStream_t s) {
  if (trans == 0) {
    const int rc = launch_sdd_rowblock(L, A, B, S, Z, K, dt, s);
    if (rc != kNotApplicable) return rc;
  }
  if (dt == BS_BF16) return run_t<bf16_t>(L, A, B, S, Z, K, trans, s);
  if (dt == BS_F16) return run_t<f16_t>(L, A, B, S, Z, K, trans, s);
  return run_t<float>(L, A, B, S, Z, K, trans, s);
}

}  // namespace bsa
