// DDS: dense = dense x sparse, right operand sparse (Triton issue 117,
// "question on blocksparse", third mode; in attention's backward,
// dV^T = dO^T P).
//   C[z, h, :, c-block] = sum over stored (h, r, c) of A[z, h, :, r-block] . S[z, k]
//
// One workgroup (4 waves) per (batch, block column), longest columns first,
// walking the column through the CSC tables (row_idx gives the A column
// block, blk_id the stored block). Output tiles (M/T x block/T) are dealt to
// the waves. A is read as 16-byte row vectors; S down its columns (T
// consecutive floats of one block row per k value). bf16: S is rounded to
// bf16 for the product, C from the fp32 accumulator. Columns with no stored
// block are written as zeros.
#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

template <typename E>
struct SCol;
template <>
struct SCol<float> {
  static __device__ __forceinline__ Frag<float> column(const float* p, int stride) {
    Frag<float> f;
#pragma unroll
    for (int q = 0; q < 4; ++q) f.v[q] = p[q * stride];
    return f;
  }
};
template <>
struct SCol<bf16_t> {
  static __device__ __forceinline__ Frag<bf16_t> column(const float* p, int stride) {
    Frag<bf16_t> f;
#pragma unroll
    for (int q = 0; q < 8; ++q) f.v[q] = to_bf16(p[q * stride]);
    return f;
  }
};

template <typename E, int BLK, int T>
__global__ __launch_bounds__(256) void k_dds(const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ row_idx,
                                             const int32_t* __restrict__ blk_id,
                                             const int32_t* __restrict__ col_order,
                                             const typename Elem<E>::storage* __restrict__ A,
                                             const float* __restrict__ S, typename Elem<E>::storage* __restrict__ C,
                                             int Z, int H, int nbr, int nbc, int M, int64_t nnz) {
  using St = typename Elem<E>::storage;
  using AccT = typename Acc<T>::type;
  constexpr int G = 64 / T, VEC = Elem<E>::VEC, KC = G * VEC, TPB = BLK / T, NR = T * T / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane % T, g = lane / T;
  // 1-D grid, batch fastest: dispatch follows the longest-first order
  // across the whole batch
  const int hc = col_order[blockIdx.x / Z];
  const int z = blockIdx.x % Z;
  const int h = hc / nbc, c = hc % nbc;
  const int e0 = col_ptr[hc], e1 = col_ptr[hc + 1];
  const int MT = M / T;
  const int64_t zh = (int64_t)z * H + h;
  const int64_t lda = (int64_t)nbr * BLK;
  for (int it = wave; it < MT * TPB; it += 4) {
    const int tm = it / TPB, tj = it % TPB;
    AccT acc = {};
    const St* a_row = A + (zh * M + tm * T + li) * lda + g * VEC;
    for (int e = e0; e < e1; ++e) {
      const int r = row_idx[e];
      const int64_t kk = blk_id[e];
      const St* pa = a_row + (int64_t)r * BLK;
      const float* ps = S + (((int64_t)z * nnz + kk) * BLK + g * VEC) * BLK + tj * T + li;
#pragma unroll
      for (int i = 0; i < BLK; i += KC) {
        Frag<E> fa, fb;
        if (i + g * VEC < BLK) {
          fa.load(pa + i);
          fb = SCol<E>::column(ps + i * BLK, BLK);
        } else {
          fa.zero();
          fb.zero();
        }
        mma_frag<T>(acc, fa, fb);
      }
    }
    St* pc = C + (zh * M + tm * T) * ((int64_t)nbc * BLK) + (int64_t)c * BLK + tj * T + li;
#pragma unroll
    for (int q = 0; q < NR; ++q) store_elem(pc + (int64_t)acc_row<T>(q, g) * nbc * BLK, acc[q]);
  }
}

template <typename E, int BLK>
int run(const bs_layout* L, const void* A, const float* S, void* C, int Z, int M, hipStream_t s) {
  using St = typename Elem<E>::storage;
  if (BLK >= 32 && M % 32 == 0) {
    constexpr int T = BLK >= 32 ? 32 : 16;
    hipLaunchKernelGGL((k_dds<E, BLK, T>), dim3(L->H * L->nbc * Z), dim3(256), 0, s, L->col_ptr, L->row_idx,
                       L->blk_id, L->col_order, (const St*)A, S, (St*)C, Z, L->H, L->nbr, L->nbc, M, L->nnz);
  } else {
    hipLaunchKernelGGL((k_dds<E, BLK, 16>), dim3(L->H * L->nbc * Z), dim3(256), 0, s, L->col_ptr, L->row_idx,
                       L->blk_id, L->col_order, (const St*)A, S, (St*)C, Z, L->H, L->nbr, L->nbc, M, L->nnz);
  }
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

template <typename E>
int run_e(const bs_layout* L, const void* A, const float* S, void* C, int Z, int M, hipStream_t s) {
  switch (L->block) {
    case 16: return run<E, 16>(L, A, S, C, Z, M, s);
    case 32: return run<E, 32>(L, A, S, C, Z, M, s);
    case 64: return run<E, 64>(L, A, S, C, Z, M, s);
    case 128: return run<E, 128>(L, A, S, C, Z, M, s);
  }
  return fail(BS_ERR_UNSUPPORTED, "block must be 16, 32, 64 or 128");
}

}  // namespace

int launch_dds(const bs_layout* L, const void* A, const float* S, void* C, int Z, int M, bs_dtype dt,
               hipStream_t s) {
  return dt == BS_BF16 ? run_e<bf16_t>(L, A, S, C, Z, M, s) : run_e<float>(L, A, S, C, Z, M, s);
}

}  // namespace bsa
