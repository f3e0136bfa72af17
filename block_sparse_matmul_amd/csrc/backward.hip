// Fused block-sparse attention backward: the exact gradient of the fused
// forward (softmax(scale Q K^T + masks) V on the layout's blocks; Triton
// issue 117, "question on blocksparse", for the three modes the gradient is
// made of; the Triton tutorial's autograd pattern of a forward kernel and a
// backward kernel), computed without writing S or P to memory.
//
// With x = scale S + masks in log2 units, lse the row log-sum-exp written by
// the forward and D_i = dO_i . O_i (equal to sum_j P_ij dP_ij):
//   P = exp2(x - lse2),  dP = dO V^T,  dS = scale P (dP - D),
//   dQ = dS K,  dK = dS^T Q,  dV = P^T dO.
// Two kernels, each with the forward's row-block layout (one lane owns one
// row of its side, 16 rows per wave, b/16 waves per workgroup, the other
// side's block staged in LDS once per step and the next block in flight in
// registers):
//  * dQ: one workgroup per (batch, head, block row), walking the row's
//    blocks (CSR). Per block: S^T = K Q^T and dP^T = V dO^T (A = K or V rows
//    from LDS, B = the wave's Q or dO rows in registers), then
//    dQ^T += K^T dS^T (A = K read transposed). It also forms D from dO and
//    O and writes it for the second kernel.
//  * dK, dV: one workgroup per (batch, head, block column), walking the
//    column's blocks (CSC). Per block: S = Q K^T and dP = dO V^T (A = Q or
//    dO rows, B = the wave's K or V rows), then dV^T += dO^T P and
//    dK^T += Q^T dS (A = dO or Q read transposed); lse and D of the block's
//    queries are staged with it.
// fp32 keeps a second, differently padded copy of each matrix read
// transposed (one 4-byte element per lane: rows 16 mod 64 bytes apart) next
// to the row-read copy (16-byte reads: rows 32 mod 256 bytes apart), both
// free of bank conflicts, where the copies fit in LDS (not for 128-blocks
// with d = 128); the 16-bit types read both ways from one copy (rows 32 mod
// 256 bytes apart: 16-byte reads and ds_read_b64_tr_b16).
// 16-bit types: P and dS are rounded to the operand type for the products,
// results from fp32 accumulators.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

constexpr float kLog2eG = 1.4426950408889634f;

template <typename E>
struct GCfg;
template <>
struct GCfg<float> {
  static constexpr int VEC = 4, KC = 16;
  typedef f32x4 Vec;
};
template <typename E>
struct GCfg16 {
  static constexpr int VEC = 8, KC = 32;
  typedef typename H16<E>::V8 Vec;
};
template <>
struct GCfg<bf16_t> : GCfg16<bf16_t> {};
template <>
struct GCfg<f16_t> : GCfg16<f16_t> {};

// LDS of one workgroup: the two staged matrices (row reads), fp32's
// transposed-read copies where they fit, and (dK dV) lse and D of the
// block's queries
template <typename E, int BLK, int D, bool DKDV>
struct GLds {
  using St = typename Elem<E>::storage;
  static constexpr bool F32 = std::is_same<E, float>::value;
  static constexpr int RSTR = D + 32 / (int)sizeof(St);  // row reads
  static constexpr int NT_COPIES = DKDV ? 2 : 1;         // matrices read transposed
  // lse and D of the block's queries (dK dV); two slots by block parity
  // with 128-blocks, whose next block is staged in halves
  static constexpr size_t STATS = DKDV ? (BLK == 128 ? 4 : 2) * BLK * sizeof(float) : 0;
  static constexpr size_t DUP_BYTES = (size_t)(2 * BLK * RSTR + NT_COPIES * BLK * (D + 4)) * sizeof(St) + STATS;
  static constexpr bool DUP = F32 && DUP_BYTES <= 160 * 1024;  // separate transposed-read copies
  static constexpr int TSTR = DUP ? D + 4 : RSTR;               // transposed reads
  static constexpr int MAT = BLK * RSTR;
  static constexpr int TMAT = DUP ? BLK * TSTR : 0;
  static constexpr int ELEMS = 2 * MAT + NT_COPIES * TMAT;
  static constexpr size_t BYTES = (size_t)ELEMS * sizeof(St) + STATS;
};

// DKDV = false: dQ (and D) over block rows; true: dK and dV over block
// columns. ptr / idx / order: the CSR tables (row_ptr, col_idx, row_order)
// or the CSC ones (col_ptr, row_idx, col_order); n_own / n_oth: block rows
// and columns of the walked side and of the other side.
template <typename E, int BLK, int D, bool CAUSAL, bool MASKED, bool DKDV>
__global__ __launch_bounds__(BLK * 4) void k_bwd(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx, const int32_t* __restrict__ order,
    const typename Elem<E>::storage* __restrict__ Q, const typename Elem<E>::storage* __restrict__ K,
    const typename Elem<E>::storage* __restrict__ V, const typename Elem<E>::storage* __restrict__ O,
    const typename Elem<E>::storage* __restrict__ dO, typename Elem<E>::storage* __restrict__ G1,
    typename Elem<E>::storage* __restrict__ G2, const float* __restrict__ lse, float* __restrict__ Dv,
    const float* __restrict__ amask, const float* __restrict__ kpmask, int Z, int H, int n_own, int n_oth, float c,
    float scale, const int32_t* __restrict__ order_h, int grouped) {
  using St = typename Elem<E>::storage;
  using Vec = typename GCfg<E>::Vec;
  using Lay = GLds<E, BLK, D, DKDV>;
  constexpr bool BF = !std::is_same<E, float>::value;
  constexpr int VEC = GCfg<E>::VEC, KC = GCfg<E>::KC;
  constexpr int NW = BLK / 16, NT = 64 * NW;
  constexpr int NQ = D / KC;             // B fragments per lane and matrix
  constexpr int KS = BLK < 64 ? BLK : 64;  // other-side rows per sub-step
  constexpr int NSUB = BLK / KS;
  constexpr int NJT = KS / 16;
  constexpr int NNT = D / 16;
  constexpr int RSTR = Lay::RSTR, TSTR = Lay::TSTR;
  constexpr int CPR = D / VEC;
  constexpr int KCH = BLK * CPR / NT;
  static_assert(KCH >= 1 && BLK * CPR % NT == 0, "staging");
  // With two sub-steps (128-blocks) the next block is staged in halves (the
  // rows of one sub-step): a half moves into registers while the current
  // block's other half is computed and into LDS once every wave is done
  // with the half it replaces. HK chunks per thread are held; one half is
  // chunks [x HK, (x + 1) HK) of the block (whole rows: NT / CPR rows per
  // chunk index divide 64).
  constexpr int HK = NSUB == 2 ? KCH / 2 : KCH;
  static_assert(NSUB == 1 || (KCH % 2 == 0 && 64 % (NT / CPR) == 0), "halves of whole rows");

  __shared__ __attribute__((aligned(16))) unsigned char smem[Lay::BYTES];
  St* const X1r = reinterpret_cast<St*>(smem);             // K (dQ) or Q (dK dV), row reads
  St* const X2r = X1r + Lay::MAT;                          // V (dQ) or dO (dK dV), row reads
  St* const X1t = Lay::DUP ? X2r + Lay::MAT : X1r;         // transposed-read copies
  St* const X2t = Lay::DUP ? X1t + Lay::TMAT : X2r;
  float* const st_lse = reinterpret_cast<float*>(smem + (size_t)Lay::ELEMS * sizeof(St));  // DKDV only
  float* const st_d = st_lse + BLK;  // slot 1 (two sub-steps): st_lse + 2 BLK, st_d + 2 BLK

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  // Which row (column): with `grouped`, XCD-aware and grouped by (batch,
  // head), the head's rows (columns) longest first, so that the other
  // side's blocks, read again by each of them, stay in the XCD's L2;
  // otherwise longest first across the whole job, batch index fastest.
  int hu, z;
  if (grouped) {
    const int unit = xcd_unit(blockIdx.x, gridDim.x);
    const int zhu = unit / n_own;
    z = zhu / H;
    hu = order_h[(zhu % H) * n_own + unit % n_own];
  } else {
    hu = order[blockIdx.x / Z];
    z = blockIdx.x % Z;
  }
  const int h = hu / n_own, u = hu % n_own;
  int k0 = ptr[hu], k1 = ptr[hu + 1];
  if constexpr (CAUSAL) trim_causal<DKDV>(idx, u, k0, k1);
  const int64_t zh = (int64_t)z * H + h;
  const int64_t Nown = (int64_t)n_own * BLK, Noth = (int64_t)n_oth * BLK;
  const int64_t Nq = DKDV ? Noth : Nown, Nk = DKDV ? Nown : Noth;
  const int own_lo = u * BLK + wave * 16;  // first own row of this wave
  const int own = own_lo + li;             // this lane's row (query for dQ, key for dK dV)

  // ---- the lane's own rows as B fragments: F1 = Q (dQ) or K (dK dV) with
  // scale*log2(e) folded in (fp32) or only its sign (16-bit, exact);
  // F2 = dO (dQ) or V (dK dV)
  Vec f1[NQ], f2[NQ];
  float cs = 1.f;
  {
    const St* p1 = (DKDV ? K : Q) + (zh * Nown + own) * D + g * VEC;
    const St* p2 = (DKDV ? V : dO) + (zh * Nown + own) * D + g * VEC;
#pragma unroll
    for (int w = 0; w < NQ; ++w) {
      f1[w] = *reinterpret_cast<const Vec*>(p1 + w * KC);
      f2[w] = *reinterpret_cast<const Vec*>(p2 + w * KC);
    }
    if constexpr (BF) {
      const float sgn = c > 0.f ? 1.f : (c < 0.f ? -1.f : 0.f);
      if (sgn != 1.f) {
#pragma unroll
        for (int w = 0; w < NQ; ++w)
#pragma unroll
          for (int e = 0; e < 8; ++e) f1[w][e] = H16<E>::cvt((float)f1[w][e] * sgn);
      }
      cs = (c == 0.f) ? 1.f : fabsf(c);
    } else {
#pragma unroll
      for (int w = 0; w < NQ; ++w) f1[w] *= c;
    }
  }
  // dQ: this lane's row statistics. lse2 = lse in log2 units, +inf for a row
  // that saw nothing (so that P = exp2(x - lse2) is 0 there); D = dO . O,
  // written out for the dK dV kernel
  float lse2_own = 0.f, d_own = 0.f;
  if constexpr (!DKDV) {
    const float l = lse[zh * Nq + own];
    lse2_own = (l == -INFINITY) ? INFINITY : l * kLog2eG;
    const St* po = O + (zh * Nq + own) * D + g * VEC;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < NQ; ++w) {
      const Vec ov = *reinterpret_cast<const Vec*>(po + w * KC);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc = fmaf((float)f2[w][e], (float)ov[e], acc);
    }
    d_own = rows4_sum(acc);
    if (g == 0) Dv[zh * Nq + own] = d_own;
  }
  // dK dV with a key-padding mask: one value per lane (its key)
  float kp_own = 0.f;
  if constexpr (DKDV && MASKED) {
    if (kpmask != nullptr) kp_own = kpmask[(int64_t)z * Nk + own] * kLog2eG;
  }

  // ---- staging (the other side's block: rows o*BLK.. of X1 and X2)
  const St* const X1g = (DKDV ? Q : K) + zh * Noth * D;
  const St* const X2g = (DKDV ? dO : V) + zh * Noth * D;
  Vec s1[HK], s2[HK];
  float s_lse = 0.f, s_d = 0.f;  // DKDV: one query's statistics per thread (tid < BLK)
  int goff[KCH], roff[KCH], toff[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int ch = tid + i * NT;
    goff[i] = (ch / CPR) * D + (ch % CPR) * VEC;
    roff[i] = (ch / CPR) * RSTR + (ch % CPR) * VEC;
    toff[i] = (ch / CPR) * TSTR + (ch % CPR) * VEC;
  }
  // chunks [x HK, x HK + HK) of the other side's block o into registers;
  // with the first of them (x = 0) the block's query statistics (dK dV)
  auto load_part = [&](int o, int x) {
    const St* a = X1g + (int64_t)o * BLK * D;
    const St* b = X2g + (int64_t)o * BLK * D;
#pragma unroll
    for (int i = 0; i < HK; ++i) {
      s1[i] = *reinterpret_cast<const Vec*>(a + goff[x * HK + i]);
      s2[i] = *reinterpret_cast<const Vec*>(b + goff[x * HK + i]);
    }
    if constexpr (DKDV) {
      if (x == 0 && tid < BLK) {
        const float l = lse[zh * Nq + (int64_t)o * BLK + tid];
        s_lse = (l == -INFINITY) ? INFINITY : l * kLog2eG;
        s_d = Dv[zh * Nq + (int64_t)o * BLK + tid];
      }
    }
  };
  // the registers of part x into LDS; the statistics into slot `slot`
  auto store_part = [&](int x, int slot) {
#pragma unroll
    for (int i = 0; i < HK; ++i) {
      const int j = x * HK + i;
      *reinterpret_cast<Vec*>(&X1r[roff[j]]) = s1[i];
      *reinterpret_cast<Vec*>(&X2r[roff[j]]) = s2[i];
      if constexpr (Lay::DUP) {
        *reinterpret_cast<Vec*>(&X1t[toff[j]]) = s1[i];
        if constexpr (DKDV) *reinterpret_cast<Vec*>(&X2t[toff[j]]) = s2[i];
      }
    }
    if constexpr (DKDV) {
      if (x == 0 && tid < BLK) {
        st_lse[2 * BLK * slot + tid] = s_lse;
        st_d[2 * BLK * slot + tid] = s_d;
      }
    }
  };

  f32x4 acc1[NNT], acc2[DKDV ? NNT : 1];
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) acc1[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < (DKDV ? NNT : 1); ++nt) acc2[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A^T-operand product acc[n] += X^T[n][rows] W[rows][own] over the KS
  // rows of a sub-step, W from registers (w[jt][rr] = element of row
  // kofs + 16 jt + 4 g + rr); X read transposed from LDS
  auto tprod = [&](f32x4* acc, const St* Xt, int kofs, const f32x4* w) {
    if constexpr (BF) {
      using HT = H16<E>;
      using V8 = typename HT::V8;
      using V4 = typename HT::V4;
      const u16* xb = &Xt[(kofs + 4 * g + (li >> 2)) * TSTR + 4 * (li & 3)];
      if constexpr (NJT >= 2) {
#pragma unroll
        for (int jp = 0; jp < NJT / 2; ++jp) {
          const V8 pb = {HT::cvt(w[2 * jp][0]),     HT::cvt(w[2 * jp][1]),     HT::cvt(w[2 * jp][2]),
                         HT::cvt(w[2 * jp][3]),     HT::cvt(w[2 * jp + 1][0]), HT::cvt(w[2 * jp + 1][1]),
                         HT::cvt(w[2 * jp + 1][2]), HT::cvt(w[2 * jp + 1][3])};
#pragma unroll
          for (int nt = 0; nt < NNT; ++nt) {
            const V4 a0 = lds_read_tr16_as<V4>(xb + (32 * jp) * TSTR + nt * 16);
            const V4 a1 = lds_read_tr16_as<V4>(xb + (32 * jp + 16) * TSTR + nt * 16);
            const V8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            acc[nt] = HT::mfma16(a, pb, acc[nt]);
          }
        }
      } else {
        const typename HT::T zb = HT::cvt(0.f);
        const V8 pb = {HT::cvt(w[0][0]), HT::cvt(w[0][1]), HT::cvt(w[0][2]), HT::cvt(w[0][3]), zb, zb, zb, zb};
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) {
          const V4 a0 = lds_read_tr16_as<V4>(xb + nt * 16);
          const V8 a = {a0[0], a0[1], a0[2], a0[3], zb, zb, zb, zb};
          acc[nt] = HT::mfma16(a, pb, acc[nt]);
        }
      }
    } else {
      const float* xb = &Xt[(kofs + 4 * g) * TSTR + li];
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int nt = 0; nt < NNT; ++nt)
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(xb[(16 * jt + rr) * TSTR + nt * 16], w[jt][rr], acc[nt], 0,
                                                           0, 0);
        __builtin_amdgcn_sched_barrier(0);  // bound the operands in flight (registers)
      }
    }
  };
  // row-operand product out[jt] = X[rows][:] F[own][:]^T for the NJT tiles
  // of a sub-step (A = X rows from LDS, B = the lane's fragments)
  auto rprod = [&](f32x4* out, const St* Xr, int kofs, const Vec* f) {
    const St* xb = &Xr[(kofs + li) * RSTR + g * VEC];
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      out[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NQ; ++w) {
        const Vec a = *reinterpret_cast<const Vec*>(xb + 16 * jt * RSTR + w * KC);
        if constexpr (BF) {
          out[jt] = H16<E>::mfma16(a, f[w], out[jt]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) out[jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], f[w][e], out[jt], 0, 0, 0);
        }
      }
      if constexpr (!BF) __builtin_amdgcn_sched_barrier(0);  // fp32: bound the operands in flight (registers)
    }
  };

  if (k0 < k1) {
    load_part(idx[k0], 0);
    if constexpr (NSUB == 2) {
      store_part(0, 0);
      load_part(idx[k0], 1);
    }
  }
  for (int kk = k0; kk < k1; ++kk) {
    const int o = idx[kk];  // the other side's block index
    const int slot = NSUB == 2 ? (kk - k0) & 1 : 0;
    __syncthreads();  // every wave is done with the previous block
    if constexpr (NSUB == 2) {
      // the second half of this block (its first half and statistics are
      // in LDS); then the first half of the next one into registers
      store_part(1, slot);
      if (kk + 1 < k1) load_part(idx[kk + 1], 0);
    } else {
      store_part(0, 0);
      __syncthreads();
      if (kk + 1 < k1) load_part(idx[kk + 1], 0);
    }
    // causal: mask element-wise on the diagonal block (the walk holds no
    // block wholly above the diagonal)
    const bool mask_block = CAUSAL && o == u;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const int kofs = sub * KS;
      if (sub == 1) {
        // every wave is done with the first half, and the second is in LDS:
        // the next block's first half replaces this one's, and its second
        // half moves into registers
        __syncthreads();
        if (kk + 1 < k1) {
          store_part(0, slot ^ 1);
          load_part(idx[kk + 1], 1);
        }
      }
      f32x4 s[NJT], dp[NJT];
      rprod(s, X1r, kofs, f1);
      rprod(dp, X2r, kofs, f2);
      // element (own, other row e = o*BLK + kofs + 16 jt + 4 g + rr)
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        const int e0 = o * BLK + kofs + 16 * jt + 4 * g;
        f32x4 mv = {0.f, 0.f, 0.f, 0.f};
        if constexpr (MASKED) {
          if constexpr (DKDV) {
            if (amask != nullptr) {
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) mv[rr] = amask[(int64_t)(e0 + rr) * Nk + own] * kLog2eG;
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) mv[rr] += kp_own;
          } else {
            if (amask != nullptr) mv = *reinterpret_cast<const f32x4*>(amask + (int64_t)own * Nk + e0);
            if (kpmask != nullptr) mv += *reinterpret_cast<const f32x4*>(kpmask + (int64_t)z * Nk + e0);
            mv *= kLog2eG;
          }
        }
        f32x4 l2, dd;
        if constexpr (DKDV) {
          l2 = *reinterpret_cast<const f32x4*>(&st_lse[2 * BLK * slot + kofs + 16 * jt + 4 * g]);
          dd = *reinterpret_cast<const f32x4*>(&st_d[2 * BLK * slot + kofs + 16 * jt + 4 * g]);
        } else {
          l2 = f32x4{lse2_own, lse2_own, lse2_own, lse2_own};
          dd = f32x4{d_own, d_own, d_own, d_own};
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          float x = fmaf(s[jt][rr], cs, mv[rr]);
          if (CAUSAL && mask_block) {
            const int q = DKDV ? e0 + rr : own, k = DKDV ? own : e0 + rr;
            if (k > q) x = -INFINITY;
          }
          const float p = __builtin_amdgcn_exp2f(x - l2[rr]);
          s[jt][rr] = p;
          dp[jt][rr] = scale * p * (dp[jt][rr] - dd[rr]);
        }
      }
      if constexpr (DKDV) {
        tprod(acc2, X2t, kofs, s);   // dV^T += dO^T P
        tprod(acc1, X1t, kofs, dp);  // dK^T += Q^T dS
      } else {
        tprod(acc1, X1t, kofs, dp);  // dQ^T += K^T dS^T
      }
    }
  }

  // ---- results: lane (g, li) holds columns 16 nt + 4 g .. of its own row
  auto write = [&](St* G, const f32x4* acc) {
    St* pg = G + (zh * Nown + own) * D + 4 * g;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) {
      if constexpr (BF) {
        using HT = H16<E>;
        *reinterpret_cast<typename HT::V4*>(pg + nt * 16) =
            typename HT::V4{HT::cvt(acc[nt][0]), HT::cvt(acc[nt][1]), HT::cvt(acc[nt][2]), HT::cvt(acc[nt][3])};
      } else {
        *reinterpret_cast<f32x4*>(pg + nt * 16) = acc[nt];
      }
    }
  };
  write(G1, acc1);
  if constexpr (DKDV) write(G2, acc2);
}

template <typename E, int BLK, int D, bool DKDV>
int launch_k(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  using St = typename Elem<E>::storage;
  const int n_own = DKDV ? L->nbc : L->nbr, n_oth = DKDV ? L->nbr : L->nbc;
  const dim3 grid(L->H * n_own * a.Z), block(BLK * 4);
  const int32_t* ptr = DKDV ? L->col_ptr : L->row_ptr;
  const int32_t* idx = DKDV ? L->row_idx : L->col_idx;
  const int32_t* order = DKDV ? L->col_order : L->row_order;
  const int32_t* order_h = DKDV ? L->col_order_h : L->row_order_h;
  // head-grouped XCD order for 16-bit operands with rows (columns) of similar
  // length, as the 16-bit forward and the row-block SDD / DSD (measured on
  // random_b128_bf16: forward plus backward 6.30 -> 5.84 ms)
  const double per_slot = (double)a.Z * (double)L->nnz / (2.0 * L->num_cus);
  const int max_len = DKDV ? L->max_col_len : L->max_row_len;
  const int grouped = (!std::is_same<E, float>::value && 4.0 * max_len <= per_slot) ? 1 : 0;
  const float c = a.scale * kLog2eG;
  const bool masked = a.am != nullptr || a.kp != nullptr;
  St* g1 = (St*)(DKDV ? a.dK : a.dQ);
  St* g2 = DKDV ? (St*)a.dV : nullptr;
#define BSA_BWD_LAUNCH(CA, MA)                                                                                     \
  hipLaunchKernelGGL((k_bwd<E, BLK, D, CA, MA, DKDV>), grid, block, 0, s, ptr, idx, order, (const St*)a.Q,        \
                     (const St*)a.K, (const St*)a.V, (const St*)a.O, (const St*)a.dO, g1, g2, a.lse, a.Dws, a.am, \
                     a.kp, a.Z, L->H, n_own, n_oth, c, a.scale, order_h, grouped)
  if (a.causal) {
    if (masked) BSA_BWD_LAUNCH(true, true);
    else BSA_BWD_LAUNCH(true, false);
  } else {
    if (masked) BSA_BWD_LAUNCH(false, true);
    else BSA_BWD_LAUNCH(false, false);
  }
#undef BSA_BWD_LAUNCH
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

template <typename E, int BLK, int D>
int run(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  static_assert(GLds<E, BLK, D, true>::BYTES <= 160 * 1024, "LDS");
  if (int rc = launch_k<E, BLK, D, false>(L, a, s)) return rc;  // dQ and D
  return launch_k<E, BLK, D, true>(L, a, s);                    // dK and dV (reads D)
}

template <typename E, int D>
int run_b(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  switch (L->block) {
    case 16: return run<E, 16, D>(L, a, s);
    case 32: return run<E, 32, D>(L, a, s);
    case 64: return run<E, 64, D>(L, a, s);
    case 128: return run<E, 128, D>(L, a, s);
  }
  return fail(BS_ERR_UNSUPPORTED, "block must be 16, 32, 64 or 128");
}

template <typename E>
int run_e(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  if (a.d == 64) return run_b<E, 64>(L, a, s);
  if (a.d == 128) return run_b<E, 128>(L, a, s);
  return fail(BS_ERR_UNSUPPORTED, "head size d must be 64 or 128");
}

// D buffer of bs_attention_bwd_noalloc: a library-owned device array, one
// copy per device for the life of the process. Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol); it passes the device address that hipGetSymbolAddress returns,
// looked up once per device with that device current.
static __device__ __align__(256) float scratch[kBwdScratchRows];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int bwd_scratch(float** out) {
  *out = nullptr;
  int dev = -1;
  BSA_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(BS_ERR_UNSUPPORTED, "device ordinal beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return BS_OK;
}

int launch_attention_bwd(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  const int rc = launch_attention_bwd_wide(L, a, s);
  if (rc != kNotApplicable) return rc;
  if (a.dt == BS_BF16) return run_e<bf16_t>(L, a, s);
  if (a.dt == BS_F16) return run_e<f16_t>(L, a, s);
  return run_e<float>(L, a, s);
}

}  // namespace bsa
