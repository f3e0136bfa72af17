// DSD: dense = sparse x dense, left operand sparse (Triton issue 117,
// "question on blocksparse", second mode; in attention O = P V).
//   C[z, h, r-block, :] = sum over stored (h, r, c) of P[z, k] . B[z, h, c-block, :]
//
// Nd = 64 or 128 runs on the fused attention's row-block kernel (P read in
// the score-register layout, B blocks staged through LDS). Other Nd take the
// kernel below: one workgroup (4 waves) per (batch, block row), longest rows
// first. The
// output tiles of the row (block/T x Nd/T) are dealt to the waves; each
// tile accumulates over every stored block of the row and over its columns.
// P is read as 16-byte row vectors; the dense operand is read down its
// columns (T consecutive elements of one row per k value, coalesced across
// lanes). 16-bit types: P is rounded to the operand type for the product,
// C from the fp32 accumulator. Rows with no stored block are written as zeros.
#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

template <typename E>
struct PFrag;
template <>
struct PFrag<float> {
  static __device__ __forceinline__ Frag<float> load(const float* p) {
    Frag<float> f;
    f.load(p);
    return f;
  }
  static __device__ __forceinline__ Frag<float> column(const float* p, int64_t stride) {
    Frag<float> f;
#pragma unroll
    for (int q = 0; q < 4; ++q) f.v[q] = p[q * stride];
    return f;
  }
};
template <typename E>
struct PFrag16 {
  using HT = H16<E>;
  // eight fp32 values rounded to the 16-bit type
  static __device__ __forceinline__ Frag<E> load(const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    Frag<E> f;
    f.v = typename HT::V8{HT::cvt(a[0]), HT::cvt(a[1]), HT::cvt(a[2]), HT::cvt(a[3]),
                          HT::cvt(b[0]), HT::cvt(b[1]), HT::cvt(b[2]), HT::cvt(b[3])};
    return f;
  }
  static __device__ __forceinline__ Frag<E> column(const u16* p, int64_t stride) {
    Frag<E> f;
#pragma unroll
    for (int q = 0; q < 8; ++q) f.v[q] = __builtin_bit_cast(typename HT::T, p[q * stride]);
    return f;
  }
};
template <>
struct PFrag<bf16_t> : PFrag16<bf16_t> {};
template <>
struct PFrag<f16_t> : PFrag16<f16_t> {};

template <typename E, int BLK, int T>
__global__ __launch_bounds__(256) void k_dsd(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                                             const int32_t* __restrict__ row_order, const float* __restrict__ P,
                                             const typename Elem<E>::storage* __restrict__ B,
                                             typename Elem<E>::storage* __restrict__ C, int Z, int H, int nbr,
                                             int nbc, int Nd, int64_t nnz) {
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
  const int NT = Nd / T;
  const int64_t zh = (int64_t)z * H + h;
  for (int it = wave; it < TPB * NT; it += 4) {
    const int ti = it / NT, tn = it % NT;
    AccT acc = {};
    for (int kk = k0; kk < k1; ++kk) {
      const int c = col_idx[kk];
      const float* pp = P + (((int64_t)z * nnz + kk) * BLK + ti * T + li) * BLK + g * VEC;
      const St* pb = B + (zh * nbc * BLK + (int64_t)c * BLK + g * VEC) * Nd + tn * T + li;
#pragma unroll
      for (int j = 0; j < BLK; j += KC) {
        Frag<E> fa, fb;
        if (j + g * VEC < BLK) {
          fa = PFrag<E>::load(pp + j);
          fb = PFrag<E>::column(pb + (int64_t)j * Nd, Nd);
        } else {
          fa.zero();
          fb.zero();
        }
        mma_frag<T>(acc, fa, fb);
      }
    }
    St* pc = C + (zh * nbr * BLK + (int64_t)r * BLK + ti * T) * Nd + tn * T + li;
#pragma unroll
    for (int q = 0; q < NR; ++q) store_elem<E>(pc + (int64_t)acc_row<T>(q, g) * Nd, acc[q]);
  }
}

template <typename E, int BLK>
int run(const bs_layout* L, const float* P, const void* B, void* C, int Z, int Nd, hipStream_t s) {
  using St = typename Elem<E>::storage;
  if (BLK >= 32 && Nd % 32 == 0) {
    constexpr int T = BLK >= 32 ? 32 : 16;
    hipLaunchKernelGGL((k_dsd<E, BLK, T>), dim3(L->H * L->nbr * Z), dim3(256), 0, s, L->row_ptr, L->col_idx,
                       L->row_order, P, (const St*)B, (St*)C, Z, L->H, L->nbr, L->nbc, Nd, L->nnz);
  } else {
    hipLaunchKernelGGL((k_dsd<E, BLK, 16>), dim3(L->H * L->nbr * Z), dim3(256), 0, s, L->row_ptr, L->col_idx,
                       L->row_order, P, (const St*)B, (St*)C, Z, L->H, L->nbr, L->nbc, Nd, L->nnz);
  }
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

template <typename E>
int run_e(const bs_layout* L, const float* P, const void* B, void* C, int Z, int Nd, hipStream_t s) {
  switch (L->block) {
    case 16: return run<E, 16>(L, P, B, C, Z, Nd, s);
    case 32: return run<E, 32>(L, P, B, C, Z, Nd, s);
    case 64: return run<E, 64>(L, P, B, C, Z, Nd, s);
    case 128: return run<E, 128>(L, P, B, C, Z, Nd, s);
  }
  return fail(BS_ERR_UNSUPPORTED, "block must be 16, 32, 64 or 128");
}

}  // namespace

int launch_dsd(const bs_layout* L, const float* P, const void* B, void* C, int Z, int Nd, bs_dtype dt,
               hipStream_t s) {
  const int rc = launch_dsd_rowblock(L, P, B, C, Z, Nd, dt, s);
  if (rc != kNotApplicable) return rc;
  if (dt == BS_BF16) return run_e<bf16_t>(L, P, B, C, Z, Nd, s);
  if (dt == BS_F16) return run_e<f16_t>(L, P, B, C, Z, Nd, s);
  return run_e<float>(L, P, B, C, Z, Nd, s);
}

}  // namespace bsa
