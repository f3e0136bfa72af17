// Fused block-sparse attention backward for 16-bit operands (bf16, fp16),
// blocks of 64 and 128, no dense masks: the gradient of backward.hip (the
// exact gradient of the fused forward; the three modes of Triton issue 117,
// "question on blocksparse"; the Triton tutorial's forward-kernel /
// backward-kernel autograd pattern), laid out like the 16-bit forward.
//
// With x = scale S in log2 units, lse the forward's row log-sum-exp and
// D_i = dO_i . O_i:  P = exp2(x - lse2), dP = dO V^T, dS = scale P (dP - D),
// dQ = dS K, dK = dS^T Q, dV = P^T dO.
//
// What differs from the 16-row kernels of backward.hip:
//  * each wave owns 32 rows of its side (two 16-row tiles), so every
//    operand read from LDS feeds two MFMAs (the 16-row kernels read the
//    whole staged block per 16 rows and were bound by LDS reads);
//  * the other side's block is staged by LDS DMA (buffer_load_dwordx4 ...
//    lds, a scalar base and a 32-bit per-lane offset) into unpadded rows
//    whose 16-byte chunks are XOR-swizzled by row, the layout of the 16-bit
//    forward: row reads (16 bytes a lane) and transposing reads
//    (ds_read_b64_tr_b16) are both free of bank conflicts;
//  * each block moves in two halves with one barrier per half; a half is
//    fetched as soon as every wave is done with the slot it refills, after
//    the first chunk's row products (so that its LDS writes do not queue
//    ahead of their reads), and every operand of a product is requested
//    before its first MFMA (scheduling barriers).
// Two kernels:
//  * dQ (k_bwd_wide): one workgroup per (batch, head, block row); per
//    32-key chunk of a column block: S^T = K Q^T and dP^T - D = V dO^T - D
//    (K, V rows from LDS, Q and dO rows of the wave in registers), P and
//    dS in registers, then dQ^T += K^T dS^T (K read transposed). It also
//    forms D and writes -D to the workspace.
//  * dK and dV (k_bwd_dkv_pipe): one workgroup per (batch, head, block
//    column) with two groups of waves on the same 32-key tiles. The dV
//    waves form S and P once per 32-query chunk, hand P to the dK waves
//    through LDS and accumulate dV^T += dO^T P; the dK waves run one
//    staged half behind: dP - D, dS, dK^T += Q^T dS. S is formed once per
//    block (14 b^2 d executed over both kernels instead of 16): a wave
//    holding both accumulators would need more than the 256 registers of
//    two waves per SIMD, and handing P over with a barrier per chunk
//    measured no faster; running the dK waves a half behind lets the one
//    barrier per half order the hand-over.
// P and dS / scale are rounded to the operand type for the products (the
// scale multiplies dQ and dK once, at the end); gradients are rounded once
// from float32 accumulators.
#include <math.h>

#include <type_traits>

#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

constexpr float kLog2eW = 1.4426950408889634f;

typedef __attribute__((address_space(3))) unsigned char lds_u8w;
// fourth word of a raw buffer resource on gfx9 (32-bit data format, no
// swizzle, no index stride)
constexpr int kRsrcWord3W = 0x00020000;

// 16-byte chunk slot of a row's chunk: d = 128 (256-byte rows): chunk ^
// ((2 row) & 14); d = 64 (128-byte rows): chunk ^ (((row >> 1) ^ row) & 7).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return (2 * r) & 14;
  else return ((r >> 1) ^ r) & 7;
}

// KP: a key-padding mask kpmask [Z][keys] (additive, natural-log units)
// joins the scores as x = s |c| + log2(e) kp, the forward's form; a dense
// attention mask takes the 16-row kernels (read once more per pass here).

// ---- dQ: own rows are the wave's 32 queries, the walk goes over the
// block row's key blocks (K and V staged)
template <typename E, int BLK, int D, bool CAUSAL, bool KP>
__global__ __launch_bounds__(BLK * 2, 2) void k_bwd_wide(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx, const int32_t* __restrict__ order,
    const int32_t* __restrict__ order_h, int grouped, const u16* __restrict__ Q, const u16* __restrict__ K,
    const u16* __restrict__ V, const u16* __restrict__ O, const u16* __restrict__ dO, u16* __restrict__ G,
    const float* __restrict__ lse, float* __restrict__ Dv, int Z, int H, int n_own, int n_oth, float c,
    float scale, const float* __restrict__ kpmask) {
  using HT = H16<E>;
  using V8 = typename HT::V8;
  using V4 = typename HT::V4;
  constexpr int NW = BLK / 32;       // waves (32 own rows each)
  constexpr int NQ = D / 32;         // 8-element fragments per row and lane
  constexpr int NNT = D / 16;        // 16-column tiles of a gradient
  constexpr int RB = 2 * D;          // bytes per row
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;     // rows per DMA instruction (64 lanes x 16 bytes)
  constexpr int HALF = BLK / 2;      // rows per staged half
  constexpr int PB = HALF * RB;      // bytes per half and matrix
  constexpr int NIP = PB / 1024 / NW;  // DMA instructions per wave, half and matrix
  constexpr int NCH = HALF / 32;     // 32-row chunks per half
  static_assert(NIP >= 1 && PB % (1024 * NW) == 0, "whole DMA instructions per wave");
  static_assert(NCH >= 1, "blocks of 64 or 128");

  __shared__ __attribute__((aligned(16))) unsigned char X1s[BLK * RB];  // K
  __shared__ __attribute__((aligned(16))) unsigned char X2s[BLK * RB];  // V

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
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
  if constexpr (CAUSAL) trim_causal<false>(idx, u, k0, k1);
  const int64_t zh = (int64_t)z * H + h;
  const int64_t Nown = (int64_t)n_own * BLK, Noth = (int64_t)n_oth * BLK;
  const int own_lo = u * BLK + wave * 32;  // first own row of this wave

  // ---- the wave's own rows (two tiles) as B fragments: F1 = Q with the
  // sign of scale*log2(e) folded in (exact), F2 = dO
  const float sgn = c > 0.f ? 1.f : (c < 0.f ? -1.f : 0.f);
  const float cs = (c == 0.f) ? 1.f : fabsf(c);
  V8 f1[2][NQ], f2[2][NQ];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const u16* p1 = Q + (zh * Nown + own_lo + 16 * t + li) * D + 8 * g;
    const u16* p2 = dO + (zh * Nown + own_lo + 16 * t + li) * D + 8 * g;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      f1[t][q] = *reinterpret_cast<const V8*>(p1 + 32 * q);
      f2[t][q] = *reinterpret_cast<const V8*>(p2 + 32 * q);
      if (sgn != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f1[t][q][e] = HT::cvt((float)f1[t][q][e] * sgn);
      }
    }
  }
  // the tiles' row statistics: lse2 = lse in log2 units (+inf for a row
  // that saw nothing, so that P = 0 there), D = dO . O, written out as -D
  // (the dK pass starts its dP accumulators from it)
  float lse2_own[2], d_own[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t row = zh * Nown + own_lo + 16 * t + li;
    const float l = lse[row];
    lse2_own[t] = (l == -INFINITY) ? INFINITY : l * kLog2eW;
    const u16* po = O + row * D + 8 * g;
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const V8 ov = *reinterpret_cast<const V8*>(po + 32 * q);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)f2[t][q][e], (float)ov[e], acc);
    }
    d_own[t] = rows4_sum(acc);
    if (g == 0) Dv[row] = -d_own[t];
  }

  // ---- DMA: instruction i of this wave moves rows (wave + NW i) * RPI .. of
  // a half; lane l fills slot l % CPR of row l / CPR with the chunk that the
  // swizzle puts there. The swizzle of a row depends only on the parity of
  // the instruction (halves start at multiples of 16 rows).
  int dofs[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int ri = lane / CPR, slot = lane % CPR;
    dofs[p] = ri * RB + ((slot ^ swz<D>(p * RPI + ri)) * 16);
  }
  const int d_even = (wave & 1) ? dofs[1] : dofs[0];
  const int d_odd = (wave & 1) ? dofs[0] : dofs[1];
  // K and V of this (batch, head) as raw buffer resources (the launch
  // checks that they fit in 32-bit offsets): each transfer takes a scalar
  // base and offset and a 32-bit per-lane offset
  const __amdgpu_buffer_rsrc_t x1res = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(K + zh * Noth * D), 0, (int)(unsigned)(Noth * RB), kRsrcWord3W);
  const __amdgpu_buffer_rsrc_t x2res = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(V + zh * Noth * D), 0, (int)(unsigned)(Noth * RB), kRsrcWord3W);
  auto dma_half = [&](int o, int x) {
    const unsigned base = (unsigned)(o * BLK + x * HALF) * (unsigned)RB;
#pragma unroll
    for (int i = 0; i < NIP; ++i) {
      const int I = wave + NW * i;  // uniform
      const unsigned off = (unsigned)(((NW * i) & 1) ? d_odd : d_even);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x1res, (lds_u8w*)(X1s + x * PB + I * 1024), 16, off,
                                               base + I * 1024, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x2res, (lds_u8w*)(X2s + x * PB + I * 1024), 16, off,
                                               base + I * 1024, 0, 0);
    }
  };

  // ---- LDS read offsets (bytes). Row reads: lane (g, li) reads row li,
  // chunk 4 q + g; transposing reads: lane (g, 4 k + m) reads row 4 g + k,
  // the 8 bytes at column 16 nt + 4 m. Row offsets that are multiples of 16
  // keep the swizzle and go into the instruction offsets.
  int roff[NQ], toff[NNT];
#pragma unroll
  for (int q = 0; q < NQ; ++q) roff[q] = li * RB + (((4 * q + g) ^ swz<D>(li)) * 16);
  {
    const int kk = li >> 2, m = li & 3, vr = 4 * g + kk;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) toff[nt] = vr * RB + (((2 * nt + (m >> 1)) ^ swz<D>(vr)) * 16) + 8 * (m & 1);
  }

  f32x4 acc[2][NNT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // out[t][jt] = init[t][jt] + X rows (16 jt + li of the chunk) . F[t]
  // rows, both tiles from one read of each X operand
  auto rprod = [&](f32x4 (&out)[2][2], const unsigned char* xb, const auto& f, const f32x4 (&init)[2][2]) {
    // the operands of tile 1 are read while tile 0 is multiplied
    V8 a[2][NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) a[0][q] = *reinterpret_cast<const V8*>(xb + roff[q]);
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      if (jt == 0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) a[1][q] = *reinterpret_cast<const V8*>(xb + 16 * RB + roff[q]);
      }
      __builtin_amdgcn_sched_barrier(0);
      out[0][jt] = init[0][jt];
      out[1][jt] = init[1][jt];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        out[0][jt] = HT::mfma16(a[jt][q], f[0][q], out[0][jt]);
        out[1][jt] = HT::mfma16(a[jt][q], f[1][q], out[1][jt]);
      }
    }
  };
  // acc[t][nt] += X^T (columns 16 nt.., the chunk's 32 rows) . W[t], W the
  // 32 rows of the chunk in the score-register layout (w[t][jt][rr]: row
  // 16 jt + 4 g + rr), rounded to the operand type; both tiles from one
  // pair of transposing reads
  auto tprod = [&](const unsigned char* xb, const f32x4 (&w)[2][2]) {
    V8 pb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      pb[t] = V8{HT::cvt(w[t][0][0]), HT::cvt(w[t][0][1]), HT::cvt(w[t][0][2]), HT::cvt(w[t][0][3]),
                 HT::cvt(w[t][1][0]), HT::cvt(w[t][1][1]), HT::cvt(w[t][1][2]), HT::cvt(w[t][1][3])};
    V4 a0[NNT], a1[NNT];
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) {
      a0[nt] = lds_read_tr16_as<V4>(reinterpret_cast<const u16*>(xb + toff[nt]));
      a1[nt] = lds_read_tr16_as<V4>(reinterpret_cast<const u16*>(xb + 16 * RB + toff[nt]));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) {
      const V8 a = {a0[nt][0], a0[nt][1], a0[nt][2], a0[nt][3], a1[nt][0], a1[nt][1], a1[nt][2], a1[nt][3]};
      acc[0][nt] = HT::mfma16(a, pb[0], acc[0][nt]);
      acc[1][nt] = HT::mfma16(a, pb[1], acc[1][nt]);
    }
  };

  // S starts from 0, dP from -D: the product then holds dP - D
  const f32x4 zero[2][2] = {};
  f32x4 nd[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) nd[t][jt] = f32x4{-d_own[t], -d_own[t], -d_own[t], -d_own[t]};

  if (k0 < k1) dma_half(idx[k0], 0);
  for (int kk = k0; kk < k1; ++kk) {
    const int o = idx[kk];  // the key block
    // causal: the diagonal block holds keys after queries (every wave of
    // the workgroup computes on it: each has some pair on or below the
    // diagonal)
    const bool mask_block = CAUSAL && o == u;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      // this half has landed (the only transfer in flight), and every wave
      // is done with the half about to be refetched
      __builtin_amdgcn_s_waitcnt(kVmcntZero);
      __syncthreads();
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int rofs = x * HALF + 32 * ch;  // first row of the chunk within the block
        const unsigned char* x1 = X1s + rofs * RB;
        const unsigned char* x2 = X2s + rofs * RB;
        f32x4 s[2][2], dp[2][2];
        // with a key-padding mask: the values of the chunk's keys (read
        // while the row products run)
        f32x4 kpv[KP ? 2 : 1];
        if constexpr (KP) {
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
            kpv[jt] = *reinterpret_cast<const f32x4*>(kpmask + (int64_t)z * Noth + o * BLK + rofs + 16 * jt + 4 * g);
        }
        rprod(s, x1, f1, zero);
        rprod(dp, x2, f2, nd);
        if (ch == 0) {
          if (x == 0) dma_half(o, 1);
          else if (kk + 1 < k1) dma_half(idx[kk + 1], 0);
        }
        // element (query 16 t + li, key rofs + 16 jt + 4 g + rr)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              float xv = s[t][jt][rr] * cs;
              if constexpr (KP) xv = fmaf(kpv[jt][rr], kLog2eW, xv);
              if (CAUSAL && mask_block) {
                const int own_r = own_lo + 16 * t + li, oth = o * BLK + rofs + 16 * jt + 4 * g + rr;
                if (oth > own_r) xv = -INFINITY;
              }
              const float p = __builtin_amdgcn_exp2f(xv - lse2_own[t]);
              dp[t][jt][rr] *= p;  // (dP - D) P = dS / scale
            }
        tprod(x1, dp);  // dQ^T += K^T dS^T
      }
    }
  }

  // ---- results: lane (g, li) holds columns 16 nt + 4 g .. of own row
  // 16 t + li; dQ takes the scale of dS here, once per element
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    u16* pg = G + (zh * Nown + own_lo + 16 * t + li) * D + 4 * g;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt)
      *reinterpret_cast<V4*>(pg + nt * 16) = V4{HT::cvt(acc[t][nt][0] * scale), HT::cvt(acc[t][nt][1] * scale),
                                                HT::cvt(acc[t][nt][2] * scale), HT::cvt(acc[t][nt][3] * scale)};
  }
}

template <typename E, int BLK, int D>
int launch_dq(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  const bool kp = a.kp != nullptr;
  const dim3 grid(L->H * L->nbr * a.Z), block(BLK * 2);
  // head-grouped XCD order with rows of similar length, as the 16-row
  // kernels (two workgroups per CU)
  const double per_slot = (double)a.Z * (double)L->nnz / (2.0 * L->num_cus);
  const int grouped = (4.0 * L->max_row_len <= per_slot) ? 1 : 0;
  const float c = a.scale * kLog2eW;
#define BSA_BWDQ_LAUNCH(CA, KPM)                                                                                 \
  hipLaunchKernelGGL((k_bwd_wide<E, BLK, D, CA, KPM>), grid, block, 0, s, L->row_ptr, L->col_idx, L->row_order,  \
                     L->row_order_h, grouped, (const u16*)a.Q, (const u16*)a.K, (const u16*)a.V, (const u16*)a.O, \
                     (const u16*)a.dO, (u16*)a.dQ, a.lse, a.Dws, a.Z, L->H, L->nbr, L->nbc, c, a.scale, a.kp)
  if (a.causal) {
    if (kp) BSA_BWDQ_LAUNCH(true, true);
    else BSA_BWDQ_LAUNCH(true, false);
  } else {
    if (kp) BSA_BWDQ_LAUNCH(false, true);
    else BSA_BWDQ_LAUNCH(false, false);
  }
#undef BSA_BWDQ_LAUNCH
  BSA_HIP(hipGetLastError());
  return BS_OK;
}


// dK and dV in one workgroup with S formed once: the dV waves (second half
// of the workgroup) form S and P for each 32-row chunk of a staged half of
// the row block, pass P (rounded to 16 bits) to the dK waves through LDS,
// and accumulate dV^T += dO^T P; the dK waves run one half behind: dP - D
// from their V rows and the staged dO rows, dS / scale = P (dP - D), and
// dK^T += Q^T dS. The staged halves of Q and dO form a ring of three
// (the dV waves' half, the dK waves' half, the one in flight), P a ring of
// two, so that one barrier per half orders every hand-over.
template <typename E, int BLK, int D, bool CAUSAL, bool KP>
__global__ __launch_bounds__(BLK * 4, 1) void k_bwd_dkv_pipe(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx, const int32_t* __restrict__ order,
    const int32_t* __restrict__ order_h, int grouped, const u16* __restrict__ Q, const u16* __restrict__ K,
    const u16* __restrict__ V, const u16* __restrict__ dO, u16* __restrict__ dK, u16* __restrict__ dVo,
    const float* __restrict__ lse, const float* __restrict__ Dv, int Z, int H, int n_own, int n_oth, float c,
    float scale, const float* __restrict__ kpmask) {
  using HT = H16<E>;
  using V8 = typename HT::V8;
  using V4 = typename HT::V4;
  constexpr int NWR = BLK / 32;     // waves per role (32 own rows each)
  constexpr int NW = 2 * NWR;       // waves of the workgroup
  constexpr int NQ = D / 32;
  constexpr int NNT = D / 16;
  constexpr int RB = 2 * D;
  constexpr int CPR = D / 8;
  constexpr int RPI = 1024 / RB;
  constexpr int HALF = BLK / 2;
  constexpr int PB = HALF * RB;      // bytes per half and matrix
  constexpr int NIP = PB / 1024 / NW;
  constexpr int NCH = HALF / 32;
  constexpr int PT = 2048;           // bytes of one wave's P tile of a chunk (32 x 32, 16 bits)
  static_assert(NIP >= 1 && PB % (1024 * NW) == 0, "whole DMA instructions per wave");
  __shared__ __attribute__((aligned(16))) unsigned char X1s[3 * PB];  // Q halves, ring of three
  __shared__ __attribute__((aligned(16))) unsigned char X2s[3 * PB];  // dO halves
  __shared__ __attribute__((aligned(16))) unsigned char Ps[2 * NCH * NWR * PT];
  __shared__ __attribute__((aligned(16))) float Ss[2][256];  // lse and -D of a row block, by parity

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
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
  if constexpr (CAUSAL) trim_causal<true>(idx, u, k0, k1);
  const int n = k1 - k0;
  const int64_t zh = (int64_t)z * H + h;
  const int64_t Nown = (int64_t)n_own * BLK, Noth = (int64_t)n_oth * BLK;
  const int role = wave / NWR;  // 0: dK, 1: dV
  const int wr = wave % NWR;
  const int own_lo = u * BLK + wr * 32;

  // own rows as B fragments: K (dV waves, sign of scale*log2(e) folded in)
  // or V (dK waves)
  const float sgn = c > 0.f ? 1.f : (c < 0.f ? -1.f : 0.f);
  const float cs = (c == 0.f) ? 1.f : fabsf(c);
  V8 fo[2][NQ];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const u16* p1 = (role ? K : V) + (zh * Nown + own_lo + 16 * t + li) * D + 8 * g;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      fo[t][q] = *reinterpret_cast<const V8*>(p1 + 32 * q);
      if (role == 1 && sgn != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) fo[t][q][e] = HT::cvt((float)fo[t][q][e] * sgn);
      }
    }
  }
  float kp_own[2] = {0.f, 0.f};
  if constexpr (KP) {
#pragma unroll
    for (int t = 0; t < 2; ++t) kp_own[t] = kpmask[(int64_t)z * Nown + own_lo + 16 * t + li];
  }

  // ---- DMA (as k_bwd_wide): instruction i of this wave moves rows
  // (wave + NW i) * RPI .. of a half
  int dofs[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int ri = lane / CPR, slot = lane % CPR;
    dofs[p] = ri * RB + ((slot ^ swz<D>(p * RPI + ri)) * 16);
  }
  const int d_even = (wave & 1) ? dofs[1] : dofs[0];
  const int d_odd = (wave & 1) ? dofs[0] : dofs[1];
  const __amdgpu_buffer_rsrc_t x1res = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(Q + zh * Noth * D), 0, (int)(unsigned)(Noth * RB), kRsrcWord3W);
  const __amdgpu_buffer_rsrc_t x2res = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>(dO + zh * Noth * D), 0, (int)(unsigned)(Noth * RB), kRsrcWord3W);
  const __amdgpu_buffer_rsrc_t lres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(lse + zh * Noth), 0, (int)(unsigned)(Noth * 4), kRsrcWord3W);
  const __amdgpu_buffer_rsrc_t dres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(Dv + zh * Noth), 0, (int)(unsigned)(Noth * 4), kRsrcWord3W);
  // half hh of the walk (block k0 + hh / 2, half hh & 1) into ring slot hh % 3
  auto dma_half = [&](int hh) {
    const int o = idx[k0 + (hh >> 1)], x = hh & 1, sl = hh % 3;
    const unsigned base = (unsigned)(o * BLK + x * HALF) * (unsigned)RB;
    if (x == 0 && wave == 0) {
      const int ch = lane < BLK / 2 ? lane : BLK / 2 - 1;
      const unsigned qofs = (unsigned)(o * BLK) * 4u;
      float* st = &Ss[(hh >> 1) & 1][0];
      if (ch < BLK / 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(lres, (lds_u8w*)st, 16, 16u * ch, qofs, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(dres, (lds_u8w*)st, 16, 16u * (ch - BLK / 4), qofs, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NIP; ++i) {
      const int I = wave + NW * i;
      const unsigned off = (unsigned)(((NW * i) & 1) ? d_odd : d_even);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x1res, (lds_u8w*)(X1s + sl * PB + I * 1024), 16, off,
                                               base + I * 1024, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(x2res, (lds_u8w*)(X2s + sl * PB + I * 1024), 16, off,
                                               base + I * 1024, 0, 0);
    }
  };

  int roff[NQ], toff[NNT];
#pragma unroll
  for (int q = 0; q < NQ; ++q) roff[q] = li * RB + (((4 * q + g) ^ swz<D>(li)) * 16);
  {
    const int kk = li >> 2, m = li & 3, vr = 4 * g + kk;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) toff[nt] = vr * RB + (((2 * nt + (m >> 1)) ^ swz<D>(vr)) * 16) + 8 * (m & 1);
  }
  f32x4 acc[2][NNT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) acc[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto rprod = [&](f32x4 (&out)[2][2], const unsigned char* xb, const f32x4 (&init)[2][2]) {
    // the operands of tile 1 are read while tile 0 is multiplied
    V8 a[2][NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) a[0][q] = *reinterpret_cast<const V8*>(xb + roff[q]);
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      if (jt == 0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) a[1][q] = *reinterpret_cast<const V8*>(xb + 16 * RB + roff[q]);
      }
      __builtin_amdgcn_sched_barrier(0);
      out[0][jt] = init[0][jt];
      out[1][jt] = init[1][jt];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        out[0][jt] = HT::mfma16(a[jt][q], fo[0][q], out[0][jt]);
        out[1][jt] = HT::mfma16(a[jt][q], fo[1][q], out[1][jt]);
      }
    }
  };
  // acc += X^T (the chunk's 32 rows) . W, W given as 16-bit B fragments
  auto tprod = [&](const unsigned char* xb, const V8 (&pb)[2]) {
    V4 a0[NNT], a1[NNT];
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) {
      a0[nt] = lds_read_tr16_as<V4>(reinterpret_cast<const u16*>(xb + toff[nt]));
      a1[nt] = lds_read_tr16_as<V4>(reinterpret_cast<const u16*>(xb + 16 * RB + toff[nt]));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) {
      const V8 a = {a0[nt][0], a0[nt][1], a0[nt][2], a0[nt][3], a1[nt][0], a1[nt][1], a1[nt][2], a1[nt][3]};
      acc[0][nt] = HT::mfma16(a, pb[0], acc[0][nt]);
      acc[1][nt] = HT::mfma16(a, pb[1], acc[1][nt]);
    }
  };
  auto pack = [&](const f32x4 (&w)[2][2], V8 (&pb)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      pb[t] = V8{HT::cvt(w[t][0][0]), HT::cvt(w[t][0][1]), HT::cvt(w[t][0][2]), HT::cvt(w[t][0][3]),
                 HT::cvt(w[t][1][0]), HT::cvt(w[t][1][1]), HT::cvt(w[t][1][2]), HT::cvt(w[t][1][3])};
  };

  // ---- the walk: step hs, for hs = 0 .. 2n: the dV waves take half hs,
  // the dK waves half hs - 1; half hs + 1 is fetched during the step
  const int last = 2 * n;  // halves 0 .. last - 1
  if (n > 0) dma_half(0);
  // one loop per role (the role dispatched outside it), so that registers
  // are allocated for each role's body alone; both meet the same barriers
  auto walk = [&](auto role_c) {
  constexpr int ROLE = decltype(role_c)::value;
  for (int hs = 0; hs <= last && n > 0; ++hs) {
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    auto issue = [&]() {
      if (hs + 1 < last) dma_half(hs + 1);
    };
    if constexpr (ROLE == 1) {
      if (hs < last) {
        const int o = idx[k0 + (hs >> 1)], x = hs & 1;
        const unsigned char* q1 = X1s + (hs % 3) * PB;
        const unsigned char* d2 = X2s + (hs % 3) * PB;
        const float* st = &Ss[(hs >> 1) & 1][0];
        const bool mask_block = CAUSAL && o == u;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
          const int rofs = x * HALF + 32 * ch;  // first row of the chunk within the block
          f32x4 l4[2];
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) l4[jt] = *reinterpret_cast<const f32x4*>(st + rofs + 16 * jt + 4 * g);
          const f32x4 zero[2][2] = {};
          f32x4 s[2][2];
          rprod(s, q1 + 32 * ch * RB, zero);
          if (ch == 0) issue();
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                float xv = s[t][jt][rr] * cs;
                if constexpr (KP) xv = fmaf(kp_own[t], kLog2eW, xv);
                const float l = l4[jt][rr];
                const float l2 = (KP && l == -INFINITY) ? INFINITY : l * kLog2eW;
                if (CAUSAL && mask_block) {
                  const int own_r = own_lo + 16 * t + li, oth = o * BLK + rofs + 16 * jt + 4 * g + rr;
                  if (own_r > oth) xv = -INFINITY;
                }
                s[t][jt][rr] = __builtin_amdgcn_exp2f(xv - l2);
              }
          V8 pb[2];
          pack(s, pb);
          // hand P to the dK wave of the same keys: two 1 KB rows of 16-byte
          // lane slots
          unsigned char* pt = Ps + (((hs & 1) * NCH + ch) * NWR + wr) * PT;
          *reinterpret_cast<V8*>(pt + 16 * lane) = pb[0];
          *reinterpret_cast<V8*>(pt + 1024 + 16 * lane) = pb[1];
          tprod(d2 + 32 * ch * RB, pb);  // dV^T += dO^T P
        }
      } else {
        issue();
      }
    } else {
      if (hs >= 1) {
        const int hp = hs - 1;
        const int x = hp & 1;
        const unsigned char* q1 = X1s + (hp % 3) * PB;
        const unsigned char* d2 = X2s + (hp % 3) * PB;
        const float* st = &Ss[(hp >> 1) & 1][0];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
          const int rofs = x * HALF + 32 * ch;
          // dP starts from -D: the product then holds dP - D
          f32x4 nd[2][2];
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(st + BLK + rofs + 16 * jt + 4 * g);
            nd[0][jt] = d4;
            nd[1][jt] = d4;
          }
          f32x4 dp[2][2];
          rprod(dp, d2 + 32 * ch * RB, nd);
          if (ch == 0) issue();
          const unsigned char* pt = Ps + (((hp & 1) * NCH + ch) * NWR + wr) * PT;
          const V8 pb0 = *reinterpret_cast<const V8*>(pt + 16 * lane);
          const V8 pb1 = *reinterpret_cast<const V8*>(pt + 1024 + 16 * lane);
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              dp[0][jt][rr] *= (float)pb0[4 * jt + rr];
              dp[1][jt][rr] *= (float)pb1[4 * jt + rr];
            }
          V8 sb[2];
          pack(dp, sb);
          tprod(q1 + 32 * ch * RB, sb);  // dK^T += Q^T dS
        }
      } else {
        issue();
      }
    }
  }
  };
  if (role == 1) walk(std::integral_constant<int, 1>{});
  else walk(std::integral_constant<int, 0>{});

  // ---- results: dK takes the scale of dS here
  const float osc = role == 0 ? scale : 1.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    u16* pg = (role == 1 ? dVo : dK) + (zh * Nown + own_lo + 16 * t + li) * D + 4 * g;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt)
      *reinterpret_cast<V4*>(pg + nt * 16) = V4{HT::cvt(acc[t][nt][0] * osc), HT::cvt(acc[t][nt][1] * osc),
                                                HT::cvt(acc[t][nt][2] * osc), HT::cvt(acc[t][nt][3] * osc)};
  }
}

template <typename E, int BLK, int D>
int launch_dkv_pipe(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  const bool kp = a.kp != nullptr;
  const dim3 grid(L->H * L->nbc * a.Z), block(BLK * 4);
  const double per_slot = (double)a.Z * (double)L->nnz / (2.0 * L->num_cus);
  const int grouped = (4.0 * L->max_col_len <= per_slot) ? 1 : 0;
  const float c = a.scale * kLog2eW;
#define BSA_DKVP_LAUNCH(CA, KPM)                                                                                 \
  hipLaunchKernelGGL((k_bwd_dkv_pipe<E, BLK, D, CA, KPM>), grid, block, 0, s, L->col_ptr, L->row_idx,             \
                     L->col_order, L->col_order_h, grouped, (const u16*)a.Q, (const u16*)a.K, (const u16*)a.V,    \
                     (const u16*)a.dO, (u16*)a.dK, (u16*)a.dV, a.lse, a.Dws, a.Z, L->H, L->nbc, L->nbr, c, a.scale, \
                     a.kp)
  if (a.causal) {
    if (kp) BSA_DKVP_LAUNCH(true, true);
    else BSA_DKVP_LAUNCH(true, false);
  } else {
    if (kp) BSA_DKVP_LAUNCH(false, true);
    else BSA_DKVP_LAUNCH(false, false);
  }
#undef BSA_DKVP_LAUNCH
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

template <typename E, int BLK, int D>
int run_w(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  if (int rc = launch_dq<E, BLK, D>(L, a, s)) return rc;  // dQ and -D
  return launch_dkv_pipe<E, BLK, D>(L, a, s);             // dK and dV (read -D)
}

template <typename E>
int run_we(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  if (L->block == 64) return a.d == 64 ? run_w<E, 64, 64>(L, a, s) : run_w<E, 64, 128>(L, a, s);
  return a.d == 64 ? run_w<E, 128, 64>(L, a, s) : run_w<E, 128, 128>(L, a, s);
}

}  // namespace

int launch_attention_bwd_wide(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  // a key-padding mask is read here; a dense attention mask, read at every
  // stored block by each of the three passes, takes the 16-row kernels
  // (two passes)
  if ((a.dt != BS_BF16 && a.dt != BS_F16) || a.am != nullptr) return kNotApplicable;
  if ((L->block != 64 && L->block != 128) || (a.d != 64 && a.d != 128)) return kNotApplicable;
  // the transfers address a (batch, head)'s matrices with 32-bit offsets
  const int64_t rows = (int64_t)(L->nbr > L->nbc ? L->nbr : L->nbc) * L->block;
  if (rows * 2 * a.d > 0xFFFFFFFFll) return kNotApplicable;
  return a.dt == BS_BF16 ? run_we<bf16_t>(L, a, s) : run_we<f16_t>(L, a, s);
}

}  // namespace bsa
