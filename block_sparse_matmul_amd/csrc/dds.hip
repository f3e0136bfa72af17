// DDS: dense = dense x sparse, right operand sparse (Triton issue 117,
// "question on blocksparse", third mode; in attention's backward,
// dV^T = dO^T P).
//   C[z, h, :, c-block] = sum over stored (h, r, c) of A[z, h, :, r-block] . S[z, k]
//
// Work decomposition. One workgroup per (batch, head, block column, 64-row
// chunk of M): grid x walks the columns longest first with the batch index
// fastest, grid y the row chunks. Four waves per key group, wave w owning
// rows 16w..16w+15 of the chunk; NS key groups deal the column's stored
// blocks among themselves and add their partial sums at the end. The
// column's stored blocks form one long contraction (block after block),
// walked in slabs of 64 rows (128 for 16 x 16 blocks, so one slab can span
// several blocks and a step always carries enough work to hide its two
// barriers): a slab is staged into LDS row-major (16-byte loads and stores,
// 16-bit types rounded on the way) and the next slab and its A fragments are already
// in flight while the current one is multiplied.
//
// The contraction runs over the rows of S, which is the strided direction
// of a row-major block; so S is the MFMA A operand, read from LDS one
// column element per lane (fp32: one 4-byte read, rows padded to 16 mod 64
// bytes; 16-bit types: two ds_read_b64_tr_b16, each 16-lane group reading a
// 4-row x 16-column patch so that every lane receives 4 rows of its own
// column), and A is the B operand, straight from global memory as 16-byte
// (fp32) or 8-byte (bf16, fp16) row vectors. With 16x16 tiles
//   C^T[j][m] += S^T[j][r] A^T[r][m]
// every lane ends up with 4 consecutive output columns of one row m, which
// it stores as one vector. 16-bit types: S rounded to the operand type (RNE)
// for the product, C
// from the fp32 accumulator. Columns with no stored block are written as
// zeros.
#include <type_traits>

#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

template <typename E>
struct Row4;  // 4 consecutive elements of an A row
template <>
struct Row4<float> {
  typedef f32x4 type;
};
template <>
struct Row4<bf16_t> {
  typedef bf16x4 type;
};
template <>
struct Row4<f16_t> {
  typedef f16x4 type;
};

template <typename E, int BLK>
struct DdsLds {
  using St = typename Elem<E>::storage;
  static constexpr bool BF = !std::is_same<E, float>::value;  // a 16-bit element type
  // contraction rows per step: the column's stored blocks are walked as one
  // long contraction (block after block), 64 rows at a time (128 for 16 x
  // 16 blocks)
  static constexpr int KS = BLK == 16 ? 128 : 64;
  static constexpr int SSTR = BF ? BLK + 16 : BLK + 4;  // padded LDS row stride (elements)
  static constexpr int SBUF = KS * SSTR;                // elements per key group
  static constexpr size_t STAGE = (size_t)SBUF * sizeof(St);
  // LDS of a workgroup with ns key groups: the stages, or the merge area
  // (4 waves x 64 lanes x BLK/4 floats per group but the first) if larger
  static constexpr size_t bytes(int ns) {
    const size_t merge = ns > 1 ? (size_t)(ns - 1) * 4 * 64 * (BLK / 4) * sizeof(float) : 0;
    return ns * STAGE > merge ? ns * STAGE : merge;
  }
};

template <typename E, int BLK, int NS>
__global__ __launch_bounds__(256 * NS) void k_dds(const int32_t* __restrict__ col_ptr,
                                                  const int32_t* __restrict__ row_idx,
                                                  const int32_t* __restrict__ blk_id,
                                                  const int32_t* __restrict__ col_order,
                                                  const typename Elem<E>::storage* __restrict__ A,
                                                  const float* __restrict__ S, typename Elem<E>::storage* __restrict__ C,
                                                  int Z, int H, int nbr, int nbc, int M, int64_t nnz) {
  using St = typename Elem<E>::storage;
  using R4 = typename Row4<E>::type;
  constexpr bool BF = DdsLds<E, BLK>::BF;
  constexpr int KS = DdsLds<E, BLK>::KS, SSTR = DdsLds<E, BLK>::SSTR, SBUF = DdsLds<E, BLK>::SBUF;
  constexpr int NKT = KS / 16;   // 16-row tiles of S per step
  constexpr int NNT = BLK / 16;  // 16-column tiles of the output block
  constexpr int CPR = BLK / 4;   // 16-byte fp32 chunks per S row
  constexpr int CHUNKS = KS * CPR;
  constexpr int KCH = CHUNKS / 256;  // chunks per thread
  static_assert(CHUNKS % 256 == 0 && 64 % CPR == 0, "a wave's chunks cover whole rows of one block");
  constexpr int SLOT = 64 * 4 * NNT;  // floats per wave for the final merge
  constexpr int MERGE_ELEMS = NS > 1 ? (NS - 1) * 4 * SLOT * 4 / (int)sizeof(St) : 0;
  constexpr int LDS_ELEMS = NS * SBUF > MERGE_ELEMS ? NS * SBUF : MERGE_ELEMS;

  __shared__ __attribute__((aligned(16))) St lds[LDS_ELEMS];

  const int sg = __builtin_amdgcn_readfirstlane(threadIdx.x / 256);  // key group
  const int tid = threadIdx.x % 256;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, li = lane & 15, g = lane >> 4;
  St* const Sg = lds + sg * SBUF;
  const int hc = col_order[blockIdx.x / Z];
  const int z = blockIdx.x % Z;
  const int h = hc / nbc, c = hc % nbc;
  const int e0 = col_ptr[hc], e1 = col_ptr[hc + 1];
  const int m_tile = blockIdx.y * 64 + wave * 16;  // first row of this wave
  const bool active = m_tile < M;                  // wave-uniform
  const int64_t zh = (int64_t)z * H + h;
  const int64_t lda = (int64_t)nbr * BLK, ldc = (int64_t)nbc * BLK;
  // this lane's A row, at the 4 columns of its lane group
  const St* a_lane = A + (zh * M + (active ? m_tile + li : 0)) * lda + 4 * g;
  const float* Sz = S + (int64_t)z * nnz * (BLK * BLK);

  // chunk i of a thread: slab row srow[i], columns from 4 * (chunk % CPR);
  // the 64 chunks of a wave lie in whole rows of one stored block
  int srow[KCH], scol[KCH], loff[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int ch = tid + i * 256;
    srow[i] = ch / CPR;
    scol[i] = (ch % CPR) * 4;
    loff[i] = srow[i] * SSTR + scol[i];
  }

  const int total_rows = (e1 - e0) * BLK;  // contraction length of the column
  f32x4 sreg[KCH];  // the next slab of S
  R4 anext[NKT];    // the next step's A fragments
  R4 acur[NKT];
  // step T covers contraction rows T*KS .. T*KS + KS - 1. Every load is
  // issued on every call (rows past the column's end read its last block
  // instead, and are neither stored nor multiplied), so that the compiler
  // counts the same loads on every path and its waits leave later loads in
  // flight (a conditional load made each wait cover every load).
  auto load_step = [&](int T) {
    const int q0 = T * KS;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      // first row of this wave's chunks (uniform), then the lane's own row
      int qw = q0 + __builtin_amdgcn_readfirstlane(srow[i]);
      int q = q0 + srow[i];
      if (qw >= total_rows) {
        qw = total_rows - BLK;
        q = qw + (srow[i] % BLK);
      }
      const int64_t k = blk_id[e0 + qw / BLK];
      // S is read once: a streaming load keeps it from displacing A
      sreg[i] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(Sz + k * (BLK * BLK) + (q % BLK) * BLK + scol[i]));
    }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const int q = min(q0 + 16 * kt, total_rows - 16);
      anext[kt] = *reinterpret_cast<const R4*>(a_lane + (int64_t)row_idx[e0 + q / BLK] * BLK + q % BLK);
    }
  };
  auto store_slab = [&](int T) {
    const int q0 = T * KS;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      if (q0 + __builtin_amdgcn_readfirstlane(srow[i]) >= total_rows) continue;
      if constexpr (BF) {
        using HT = H16<E>;
        *reinterpret_cast<typename HT::V4*>(&Sg[loff[i]]) = typename HT::V4{
            HT::cvt(sreg[i][0]), HT::cvt(sreg[i][1]), HT::cvt(sreg[i][2]), HT::cvt(sreg[i][3])};
      } else {
        *reinterpret_cast<f32x4*>(&Sg[loff[i]]) = sreg[i];
      }
    }
  };

  f32x4 o[NNT];
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int total = (total_rows + KS - 1) / KS;  // steps of the column
  const int nsteps = (total + NS - 1) / NS;
  if (total > 0) load_step(sg < total ? sg : total - 1);
  for (int step = 0; step < nsteps; ++step) {
    const int t = step * NS + sg;
    const bool valid = t < total;
    __syncthreads();  // every wave is done with the previous slab in LDS
    if (valid) store_slab(t);
    __syncthreads();
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) acur[kt] = anext[kt];
    __builtin_amdgcn_sched_barrier(0);  // the copies before the next loads
    load_step(t + NS < total ? t + NS : total - 1);
    if (!valid || !active) continue;
    // 16-row tiles of this step inside the contraction (the last step of a
    // column can be partial)
    const int nkt = min(NKT, (total_rows - t * KS) / 16);

    if constexpr (BF) {
      // lane (g, 4k + q) points at row 4g + k, columns 4q.. of an n-tile and
      // receives rows 4g + 0..3 of column li
      using HT = H16<E>;
      using V8 = typename HT::V8;
      using V4 = typename HT::V4;
      const u16* sb = &Sg[(4 * g + (li >> 2)) * SSTR + 4 * (li & 3)];
      const typename HT::T zb = HT::cvt(0.f);
      const V4 z4 = {zb, zb, zb, zb};
      // tiles 2jp and 2jp+1 in one 32-deep product; a lone last tile is
      // padded with zeros
      auto pair_step = [&](int jp, bool full) {
        const V4 b1 = full ? acur[2 * jp + 1] : z4;
        const V8 b = {acur[2 * jp][0], acur[2 * jp][1], acur[2 * jp][2], acur[2 * jp][3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) {
          const V4 a0 = lds_read_tr16_as<V4>(sb + (32 * jp) * SSTR + nt * 16);
          const V4 a1 = full ? lds_read_tr16_as<V4>(sb + (32 * jp + 16) * SSTR + nt * 16) : z4;
          const V8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          o[nt] = HT::mfma16(a, b, o[nt]);
        }
      };
#pragma unroll
      for (int jp = 0; jp < NKT / 2; ++jp) {
        if (2 * jp + 1 < nkt)
          pair_step(jp, true);
        else if (2 * jp < nkt)
          pair_step(jp, false);
      }
    } else {
      // one S element per lane and instruction; tile kt+1 is read while
      // tile kt is multiplied
      const float* sb = &Sg[4 * g * SSTR + li];
      float sa[2][4][NNT];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) sa[0][rr][nt] = sb[rr * SSTR + nt * 16];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        if (kt >= nkt) break;
        if (kt + 1 < nkt) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) sa[(kt + 1) & 1][rr][nt] = sb[(16 * (kt + 1) + rr) * SSTR + nt * 16];
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int nt = 0; nt < NNT; ++nt)
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(sa[kt & 1][rr][nt], acur[kt][rr], o[nt], 0, 0, 0);
      }
    }
  }

  // ---- add the key groups' partial sums into group 0 through LDS
  if constexpr (NS > 1) {
    float* red = reinterpret_cast<float*>(lds);
    __syncthreads();
    if (sg > 0) {
      float* slot = red + ((sg - 1) * 4 + wave) * SLOT;
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) slot[(nt * 4 + e) * 64 + lane] = o[nt][e];
    }
    __syncthreads();
    if (sg > 0) return;
#pragma unroll
    for (int s2 = 1; s2 < NS; ++s2) {
      const float* slot = red + ((s2 - 1) * 4 + wave) * SLOT;
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[nt][e] += slot[(nt * 4 + e) * 64 + lane];
    }
  }
  if (!active) return;

  // lane (g, li) holds output columns 16 nt + 4 g + 0..3 of row m_tile + li
  St* pc = C + (zh * M + m_tile + li) * ldc + (int64_t)c * BLK + 4 * g;
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) {
    if constexpr (BF) {
      using HT = H16<E>;
      *reinterpret_cast<typename HT::V4*>(pc + nt * 16) =
          typename HT::V4{HT::cvt(o[nt][0]), HT::cvt(o[nt][1]), HT::cvt(o[nt][2]), HT::cvt(o[nt][3])};
    } else {
      *reinterpret_cast<f32x4*>(pc + nt * 16) = o[nt];
    }
  }
}

template <typename E, int BLK, int NS>
int launch_ns(const bs_layout* L, const void* A, const float* S, void* C, int Z, int M, hipStream_t s) {
  using St = typename Elem<E>::storage;
  const dim3 grid(L->H * L->nbc * Z, (M + 63) / 64), block(256 * NS);
  hipLaunchKernelGGL((k_dds<E, BLK, NS>), grid, block, 0, s, L->col_ptr, L->row_idx, L->blk_id, L->col_order,
                     (const St*)A, S, (St*)C, Z, L->H, L->nbr, L->nbc, M, L->nnz);
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

// Key groups per workgroup, chosen as for the row-wise kernels: split the
// longest column once its time alone (about four workgroups share a CU)
// exceeds a CU's share of the whole job.
template <typename E, int BLK>
int run(const bs_layout* L, const void* A, const float* S, void* C, int Z, int M, hipStream_t s) {
  using Lds = DdsLds<E, BLK>;
  constexpr int max_ns = Lds::bytes(4) <= 160 * 1024 ? 4 : (Lds::bytes(2) <= 160 * 1024 ? 2 : 1);
  const double per_cu = (double)Z * (double)L->nnz * ((M + 63) / 64) / L->num_cus;
  int ns = 1;
  while (ns < max_ns && 4.0 * L->max_col_len / ns > per_cu) ns *= 2;
  if constexpr (max_ns >= 4) {
    if (ns >= 4) return launch_ns<E, BLK, 4>(L, A, S, C, Z, M, s);
  }
  if constexpr (max_ns >= 2) {
    if (ns >= 2) return launch_ns<E, BLK, 2>(L, A, S, C, Z, M, s);
  }
  return launch_ns<E, BLK, 1>(L, A, S, C, Z, M, s);
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
  if ((M + 63) / 64 > 65535) return fail(BS_ERR_SHAPE, "M must be at most 65535*64 for the DDS");
  if (dt == BS_BF16) return run_e<bf16_t>(L, A, S, C, Z, M, s);
  if (dt == BS_F16) return run_e<f16_t>(L, A, S, C, Z, M, s);
  return run_e<float>(L, A, S, C, Z, M, s);
}

}  // namespace bsa
