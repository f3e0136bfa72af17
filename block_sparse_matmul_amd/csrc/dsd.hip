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
#include <type_traits>

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

// P^T fragments: eight (16-bit) or four (fp32) fp32 values p[0], p[s], ...
// of a block read down a column, rounded to the operand type
template <typename E>
__device__ __forceinline__ Frag<E> p_column(const float* p, int64_t s) {
  Frag<E> f;
  if constexpr (std::is_same<E, float>::value) {
    f.load_strided(p, s);
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) f.v[q] = H16<E>::cvt(p[q * s]);
  }
  return f;
}

// The general sparse x dense product, every operand addressed through
// strides, which covers each DSD and DDS with operands stored either way
// round:
//   C(u-block row i, n) = sum over the unit's stored blocks of
//                         P'(i, j) . B(o-block row j, n)
// walking a block row (TP = false: CSR tables, P' = the block) or a block
// column (TP = true: CSC tables, P' = the block transposed), o being the
// block's other index. B(j, n) is B[j * ldb + n] (BT = false) or
// B[n * ldb + j] (BT = true); C(i, n) is C[i * ldc + n] (CT = false) or
// C[n * ldc + i] (CT = true); b_head / c_head are the (batch, head) strides.
// One workgroup (4 waves) per (batch, head, unit), the unit's T x T output
// tiles dealt to the waves; N (output width) a multiple of T.
template <typename E, int BLK, int T, bool TP, bool BT, bool CT>
__global__ __launch_bounds__(256) void k_dsd_g(const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
                                               const int32_t* __restrict__ order, const int32_t* __restrict__ blk_id,
                                               const float* __restrict__ P,
                                               const typename Elem<E>::storage* __restrict__ B,
                                               typename Elem<E>::storage* __restrict__ C, int Z, int H, int n_units,
                                               int N, int64_t nnz, int64_t ldb, int64_t b_head, int64_t ldc,
                                               int64_t c_head) {
  using St = typename Elem<E>::storage;
  using AccT = typename Acc<T>::type;
  constexpr int G = 64 / T, VEC = Elem<E>::VEC, KC = G * VEC, TPB = BLK / T, NR = T * T / 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane % T, g = lane / T;
  const int hu = order[blockIdx.x / Z];
  const int z = blockIdx.x % Z;
  const int h = hu / n_units, u = hu % n_units;
  const int k0 = ptr[hu], k1 = ptr[hu + 1];
  const int NT = N / T;
  const int64_t zh = (int64_t)z * H + h;
  const St* Bz = B + zh * b_head;
  St* Cz = C + zh * c_head;
  for (int it = wave; it < TPB * NT; it += 4) {
    const int ti = it / NT, tn = it % NT;
    const int n = tn * T + li;  // this lane's output column (B operand)
    AccT acc = {};
    for (int kk = k0; kk < k1; ++kk) {
      const int o = idx[kk];
      const int64_t blk = TP ? (int64_t)blk_id[kk] : (int64_t)kk;
      const float* pblk = P + ((int64_t)z * nnz + blk) * (BLK * BLK);
      const int64_t jrow = (int64_t)o * BLK + g * VEC;  // first B row of this lane's fragment
#pragma unroll
      for (int j = 0; j < BLK; j += KC) {
        Frag<E> fa, fb;
        if (j + g * VEC < BLK) {
          const int i = ti * T + li;  // this lane's row of P'
          if constexpr (TP) fa = p_column<E>(pblk + (int64_t)(j + g * VEC) * BLK + i, BLK);
          else fa = PFrag<E>::load(pblk + (int64_t)i * BLK + j + g * VEC);
          if constexpr (BT) fb.load(Bz + (int64_t)n * ldb + jrow + j);
          else fb.load_strided(Bz + (jrow + j) * ldb + n, ldb);
        } else {
          fa.zero();
          fb.zero();
        }
        mma_frag<T>(acc, fa, fb);
      }
    }
    const int64_t i0 = (int64_t)u * BLK + ti * T;
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int64_t i = i0 + acc_row<T>(q, g);
      store_elem<E>(CT ? Cz + (int64_t)n * ldc + i : Cz + i * ldc + n, acc[q]);
    }
  }
}

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

namespace {

template <typename E, int BLK, bool TP, bool BT, bool CT>
int run_g(const bs_layout* L, const GenArgs& a, hipStream_t s) {
  using St = typename Elem<E>::storage;
  const int n_units = TP ? L->nbc : L->nbr;
  const int32_t* ptr = TP ? L->col_ptr : L->row_ptr;
  const int32_t* idx = TP ? L->row_idx : L->col_idx;
  const int32_t* order = TP ? L->col_order : L->row_order;
  const dim3 grid(L->H * n_units * a.Z), block(256);
  if (BLK >= 32 && a.N % 32 == 0)
    hipLaunchKernelGGL((k_dsd_g<E, BLK, (BLK >= 32 ? 32 : 16), TP, BT, CT>), grid, block, 0, s, ptr, idx, order,
                       L->blk_id, a.P, (const St*)a.B, (St*)a.C, a.Z, L->H, n_units, a.N, L->nnz, a.ldb, a.b_head,
                       a.ldc, a.c_head);
  else
    hipLaunchKernelGGL((k_dsd_g<E, BLK, 16, TP, BT, CT>), grid, block, 0, s, ptr, idx, order, L->blk_id, a.P,
                       (const St*)a.B, (St*)a.C, a.Z, L->H, n_units, a.N, L->nnz, a.ldb, a.b_head, a.ldc, a.c_head);
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

template <typename E, bool TP, bool BT, bool CT>
int run_gb(const bs_layout* L, const GenArgs& a, hipStream_t s) {
  switch (L->block) {
    case 16: return run_g<E, 16, TP, BT, CT>(L, a, s);
    case 32: return run_g<E, 32, TP, BT, CT>(L, a, s);
    case 64: return run_g<E, 64, TP, BT, CT>(L, a, s);
    case 128: return run_g<E, 128, TP, BT, CT>(L, a, s);
  }
  return fail(BS_ERR_UNSUPPORTED, "block must be 16, 32, 64 or 128");
}

template <typename E>
int run_gt(const bs_layout* L, const GenArgs& a, hipStream_t s) {
  const int sel = (a.TP ? 4 : 0) | (a.BT ? 2 : 0) | (a.CT ? 1 : 0);
  switch (sel) {
    case 0: return run_gb<E, false, false, false>(L, a, s);
    case 1: return run_gb<E, false, false, true>(L, a, s);
    case 2: return run_gb<E, false, true, false>(L, a, s);
    case 3: return run_gb<E, false, true, true>(L, a, s);
    case 4: return run_gb<E, true, false, false>(L, a, s);
    case 5: return run_gb<E, true, false, true>(L, a, s);
    case 6: return run_gb<E, true, true, false>(L, a, s);
  }
  return run_gb<E, true, true, true>(L, a, s);
}

int launch_general(const bs_layout* L, const GenArgs& a, bs_dtype dt, hipStream_t s) {
  if (dt == BS_BF16) return run_gt<bf16_t>(L, a, s);
  if (dt == BS_F16) return run_gt<f16_t>(L, a, s);
  return run_gt<float>(L, a, s);
}

}  // namespace

int launch_dsd_ex(const bs_layout* L, const float* P, const void* B, void* C, int Z, int Nd, int trans, bs_dtype dt,
                  hipStream_t s) {
  const bool ta = trans & BS_TRANS_A, tb = trans & BS_TRANS_B;
  if (!ta && !tb) return launch_dsd(L, P, B, C, Z, Nd, dt, s);
  if (ta && !tb && (Nd == 64 || Nd == 128)) return launch_dsd_t(L, P, B, C, Z, Nd, dt, s);
  // rows of B: the other side of the walk (columns for the plain DSD, rows
  // for the transposed block matrix); rows of C: the walked side
  const int64_t nb_rows = (int64_t)(ta ? L->nbr : L->nbc) * L->block;
  const int64_t nc_rows = (int64_t)(ta ? L->nbc : L->nbr) * L->block;
  GenArgs a;
  a.P = P;
  a.B = B;
  a.C = C;
  a.Z = Z;
  a.N = Nd;
  a.TP = ta;
  a.BT = tb;
  a.CT = false;
  a.ldb = tb ? nb_rows : Nd;
  a.b_head = nb_rows * Nd;
  a.ldc = Nd;
  a.c_head = nc_rows * Nd;
  return launch_general(L, a, dt, s);
}

int launch_dds_ex(const bs_layout* L, const void* A, const float* S, void* C, int Z, int M, int trans, bs_dtype dt,
                  hipStream_t s) {
  const bool ta = trans & BS_TRANS_A, tb = trans & BS_TRANS_B;
  if (!ta && !tb) return launch_dds(L, A, S, C, Z, M, dt, s);
  // C^T = S'^T A^T: the walk is over block columns of S' (S' = S: CSC and
  // the blocks transposed; S' = S^T: CSR and the blocks as stored), A read
  // as the dense operand B(j, m) = A[m][j] (or A[j][m] when stored
  // transposed), C written transposed
  const int64_t na = (int64_t)(tb ? L->nbc : L->nbr) * L->block;  // A's contraction length
  const int64_t nc = (int64_t)(tb ? L->nbr : L->nbc) * L->block;  // C's columns
  GenArgs a;
  a.P = S;
  a.B = A;
  a.C = C;
  a.Z = Z;
  a.N = M;
  a.TP = !tb;
  a.BT = !ta;
  a.CT = true;
  a.ldb = ta ? M : na;
  a.b_head = na * M;
  a.ldc = nc;
  a.c_head = nc * M;
  return launch_general(L, a, dt, s);
}

}  // namespace bsa
