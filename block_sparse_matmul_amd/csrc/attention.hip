// Fused block-sparse attention: SDD -> block-sparse softmax -> DSD in one
// kernel (the composition of Triton issue 117, "question on blocksparse"),
// with the streaming softmax of the Triton tutorial (Puzzle 8, online
// softmax; Puzzle 9, simple FlashAttention): a running row max m and sum l,
// the old partial output rescaled by exp(m_old - m_new) when the max grows,
// and one division by l at the end (the same value as normalising at every
// step).
//
// Work decomposition: one workgroup per (batch, head, block row), block
// rows longest first; one wave per T query rows of the block (T = 32, or 16
// for 16-blocks). Per stored block c of the row:
//   S^T = K_c Q^T          MFMA, K rows as A, the wave's Q rows (held in
//                          registers for the whole row) as B. In the
//                          accumulator layout every lane then owns ONE query
//                          row (its column) and a slice of the keys, so the
//                          row max and sum need only in-lane work plus a
//                          butterfly across the G = 64/T lane groups.
//   online softmax         scale*log2(e) folded into one multiply, causal
//                          mask on blocks that reach the diagonal, exp2.
//   O^T += V_c^T P^T       MFMA with P^T straight from the score registers
//                          (B operand, no transpose through LDS) and V read
//                          down its columns; O^T also keeps one query row per
//                          lane, so the rescale by exp(m_old - m_new) is a
//                          per-lane scalar.
// bf16: scores, softmax and O accumulate in fp32; P is rounded to bf16
// (round-to-nearest-even) for the P.V product; O is rounded once at the end.
#include <math.h>

#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// V^T operand for one P.V instruction: the V entries (key rows, column n)
// that pair with the k values this lane's P^T fragment holds.
template <typename E, int T, int BLK>
struct PV;

template <int T, int BLK>
struct PV<float, T, BLK> {
  using AccT = typename Acc<T>::type;
  static constexpr int NR = T * T / 64;
  // o[n-tile] += V^T[n][keys of reg q] * P^T[keys of reg q][query]
  static __device__ __forceinline__ void run(AccT& o, const AccT (&p)[BLK / T], const float* pv, int D, int g) {
#pragma unroll
    for (int jt = 0; jt < BLK / T; ++jt)
#pragma unroll
      for (int q = 0; q < NR; ++q) mma(o, pv[(jt * T + acc_row<T>(q, g)) * D], p[jt][q]);
  }
};

template <int BLK>
struct PV<bf16_t, 32, BLK> {
  using AccT = f32x16;
  // each instruction takes 8 consecutive score registers (16 keys per pair of
  // instructions per 32-key tile)
  static __device__ __forceinline__ void run(AccT& o, const AccT (&p)[BLK / 32], const u16* pv, int D, int g) {
#pragma unroll
    for (int jt = 0; jt < BLK / 32; ++jt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 a, b;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          b[q] = to_bf16(p[jt][8 * u + q]);
          a[q] = __builtin_bit_cast(__bf16, pv[(jt * 32 + acc_row<32>(8 * u + q, g)) * D]);
        }
        mma(o, a, b);
      }
  }
};

template <int BLK>
struct PV<bf16_t, 16, BLK> {
  using AccT = f32x4;
  // each instruction takes the 4 score registers of two 16-key tiles
  static __device__ __forceinline__ void run(AccT& o, const AccT (&p)[BLK / 16], const u16* pv, int D, int g) {
    constexpr int NJT = BLK / 16;
#pragma unroll
    for (int jt = 0; jt < NJT; jt += 2) {
      bf16x8 a, b;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int t = jt + q / 4;
        if (t < NJT) {
          b[q] = to_bf16(p[t][q % 4]);
          a[q] = __builtin_bit_cast(__bf16, pv[(t * 16 + acc_row<16>(q % 4, g)) * D]);
        } else {
          b[q] = (__bf16)0.f;
          a[q] = (__bf16)0.f;
        }
      }
      mma(o, a, b);
    }
  }
};

template <typename E, int BLK, int T, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * (BLK / T)) void k_attn(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, const int32_t* __restrict__ row_order,
    const typename Elem<E>::storage* __restrict__ Q, const typename Elem<E>::storage* __restrict__ K,
    const typename Elem<E>::storage* __restrict__ V, typename Elem<E>::storage* __restrict__ O, int H, int nbr,
    int nbc, float c) {
  using St = typename Elem<E>::storage;
  using AccT = typename Acc<T>::type;
  constexpr int G = 64 / T, VEC = Elem<E>::VEC, KC = G * VEC, NQ = D / KC, NR = T * T / 64;
  constexpr int NJT = BLK / T, NNT = D / T;
  const float NEG = -INFINITY;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane % T, g = lane / T;
  const int hr = row_order[blockIdx.x];
  const int z = blockIdx.y;
  const int h = hr / nbr, r = hr % nbr;
  const int k0 = row_ptr[hr], k1 = row_ptr[hr + 1];
  const int64_t zh = (int64_t)z * H + h;
  const int64_t Nq = (int64_t)nbr * BLK, Nk = (int64_t)nbc * BLK;
  const int q_index = r * BLK + wave * T + li;  // this lane's query row

  // the wave's Q rows as B fragments (k values permuted per 16-byte vector)
  Frag<E> qf[NQ];
  {
    const St* pq = Q + (zh * Nq + q_index) * D + g * VEC;
#pragma unroll
    for (int u = 0; u < NQ; ++u) qf[u].load(pq + u * KC);
  }

  float m_run = NEG, l_run = 0.f;
  AccT o[NNT];
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) o[nt] = AccT{};

  for (int kk = k0; kk < k1; ++kk) {
    const int cb = col_idx[kk];
    const St* pk = K + (zh * Nk + (int64_t)cb * BLK + li) * D + g * VEC;
    const St* pv = V + (zh * Nk + (int64_t)cb * BLK) * D;

    // S^T tiles: s[jt][q] = score(query li, key jt*T + acc_row(q, g))
    AccT s[NJT];
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      s[jt] = AccT{};
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        Frag<E> kf;
        kf.load(pk + (int64_t)jt * T * D + u * KC);
        mma_frag<T>(s[jt], kf, qf[u]);
      }
    }

    // scale (log2 domain), mask, running max
    const bool mask_block = CAUSAL && (cb * BLK + BLK - 1 > r * BLK + wave * T);
    float mx = NEG;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        float x = s[jt][q] * c;
        if (mask_block && cb * BLK + jt * T + acc_row<T>(q, g) > q_index) x = NEG;
        s[jt][q] = x;
        mx = fmaxf(mx, x);
      }
#pragma unroll
    for (int off = T; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = (m_new == NEG) ? 1.f : exp2f(m_run - m_new);
    const float m_sub = (m_new == NEG) ? 0.f : m_new;
    float ls = 0.f;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
      for (int q = 0; q < NR; ++q) {
        const float pr = exp2f(s[jt][q] - m_sub);
        s[jt][q] = pr;
        ls += pr;
      }
    l_run = l_run * alpha + ls;
    m_run = m_new;

    // O^T[n][query] = alpha * O^T + V^T[n][keys] P^T[keys][query]
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) {
      o[nt] *= alpha;
      PV<E, T, BLK>::run(o[nt], s, pv + nt * T + li, D, g);
    }
  }

  // finish: l over the lane groups, O = O^T / l, written row-wise
#pragma unroll
  for (int off = T; off < 64; off <<= 1) l_run += __shfl_xor(l_run, off);
  const float inv = (l_run > 0.f) ? 1.0f / l_run : 0.f;
  St* po = O + (zh * Nq + q_index) * D;
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
    for (int q = 0; q < NR; q += 4) {
      const int n = nt * T + acc_row<T>(q, g);  // 4 consecutive columns
      if constexpr (sizeof(St) == 4) {
        *reinterpret_cast<f32x4*>(po + n) =
            f32x4{o[nt][q] * inv, o[nt][q + 1] * inv, o[nt][q + 2] * inv, o[nt][q + 3] * inv};
      } else {
        *reinterpret_cast<bf16x4*>(po + n) = bf16x4{to_bf16(o[nt][q] * inv), to_bf16(o[nt][q + 1] * inv),
                                                    to_bf16(o[nt][q + 2] * inv), to_bf16(o[nt][q + 3] * inv)};
      }
    }
}

template <typename E, int BLK, int D>
int run(const bs_layout* L, const void* Q, const void* K, const void* V, void* O, int Z, float c, bool causal,
        hipStream_t s) {
  using St = typename Elem<E>::storage;
  constexpr int T = BLK >= 32 ? 32 : 16;
  const dim3 grid(L->H * L->nbr, Z), block(64 * (BLK / T));
  if (causal)
    hipLaunchKernelGGL((k_attn<E, BLK, T, D, true>), grid, block, 0, s, L->row_ptr, L->col_idx, L->row_order,
                       (const St*)Q, (const St*)K, (const St*)V, (St*)O, L->H, L->nbr, L->nbc, c);
  else
    hipLaunchKernelGGL((k_attn<E, BLK, T, D, false>), grid, block, 0, s, L->row_ptr, L->col_idx, L->row_order,
                       (const St*)Q, (const St*)K, (const St*)V, (St*)O, L->H, L->nbr, L->nbc, c);
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

template <typename E, int D>
int run_b(const bs_layout* L, const void* Q, const void* K, const void* V, void* O, int Z, float c, bool causal,
          hipStream_t s) {
  switch (L->block) {
    case 16: return run<E, 16, D>(L, Q, K, V, O, Z, c, causal, s);
    case 32: return run<E, 32, D>(L, Q, K, V, O, Z, c, causal, s);
    case 64: return run<E, 64, D>(L, Q, K, V, O, Z, c, causal, s);
    case 128: return run<E, 128, D>(L, Q, K, V, O, Z, c, causal, s);
  }
  return fail(BS_ERR_UNSUPPORTED, "block must be 16, 32, 64 or 128");
}

template <typename E>
int run_e(const bs_layout* L, const void* Q, const void* K, const void* V, void* O, int Z, int d, float c,
          bool causal, hipStream_t s) {
  if (d == 64) return run_b<E, 64>(L, Q, K, V, O, Z, c, causal, s);
  return run_b<E, 128>(L, Q, K, V, O, Z, c, causal, s);
}

}  // namespace

int launch_attention(const bs_layout* L, const void* Q, const void* K, const void* V, void* O, int Z, int d,
                     float scale, bool causal, bs_dtype dt, hipStream_t s) {
  const float c = scale * kLog2e;
  return dt == BS_BF16 ? run_e<bf16_t>(L, Q, K, V, O, Z, d, c, causal, s)
                       : run_e<float>(L, Q, K, V, O, Z, d, c, causal, s);
}

}  // namespace bsa
