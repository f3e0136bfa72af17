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
//  * each block moves in two halves; a half is fetched as soon as every
//    wave is done with the half it replaces, and lands while the other
//    half is computed (one barrier per half). The fetch is issued after the
//    first chunk's row products, so that its LDS writes do not queue ahead
//    of their reads, and every operand of a product is requested before
//    its first MFMA (scheduling barriers): together 2% faster on
//    random_b128_bf16 (forward plus backward 4.94 against 5.03 ms).
// Work of the waves (modes of one template):
//  * dQ: one workgroup per (batch, head, block row); per 32-key chunk of a
//    column block: S^T = K Q^T and dP^T = V dO^T (K, V rows from LDS, Q and
//    dO rows of the wave in registers), P and dS in registers, then
//    dQ^T += K^T dS^T (K read transposed). It also forms D and writes it.
//  * dK: per block column; per 32-query chunk of a row block: S = Q K^T and
//    dP = dO V^T (Q, dO rows from LDS, K and V rows of the wave in
//    registers), dS with the chunk's lse and D, then dK^T += Q^T dS (Q read
//    transposed).
//  * dV: the same walk; S = Q K^T, P with the chunk's lse, then
//    dV^T += dO^T P (dO read transposed).
// Two kernels: dQ, and dK with dV in one workgroup of twice the waves
// (MODE_DKV), half of them doing the dK work and half the dV work on the
// same staged blocks of Q and dO. A wave holding both accumulators (32 rows
// x d x 2 floats) would need more than the 256 registers of two waves per
// SIMD (at one wave per SIMD it ran 8% slower than the 16-row kernel), so
// S is formed by both halves; against separate dK and dV kernels the shared
// staging measured 3-5% faster on the whole backward, bit-identical.
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

enum { MODE_DQ = 0, MODE_DK = 1, MODE_DV = 2, MODE_DKV = 3 };

// KP: a key-padding mask kpmask [Z][keys] (additive, natural-log units)
// joins the scores as x = s |c| + log2(e) kp, the forward's form; a dense
// attention mask takes the 16-row kernels (read once more per pass here).
//
// MODE_DKV: dK and dV in one workgroup of twice the waves, the first half
// accumulating dK (the dK mode's work), the second dV (the dV mode's); the
// two share each staged block of Q and dO, so the column's blocks are
// staged once instead of twice.
template <typename E, int BLK, int D, bool CAUSAL, int MODE, bool KP = false>
__global__ __launch_bounds__(BLK * 2 * (MODE == MODE_DKV ? 2 : 1), MODE == MODE_DKV ? 1 : 2) void k_bwd_wide(
    const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx, const int32_t* __restrict__ order,
    const int32_t* __restrict__ order_h, int grouped, const u16* __restrict__ Q, const u16* __restrict__ K,
    const u16* __restrict__ V, const u16* __restrict__ O, const u16* __restrict__ dO, u16* __restrict__ G,
    const float* __restrict__ lse, float* __restrict__ Dv, int Z, int H, int n_own, int n_oth, float c,
    float scale, const float* __restrict__ kpmask = nullptr, u16* __restrict__ G2 = nullptr) {
  constexpr bool DKDV = MODE != MODE_DQ;  // own rows are keys (block columns walked)
  constexpr bool DUAL = MODE == MODE_DKV;
  constexpr bool HASDP = MODE != MODE_DV;  // dP (and D) needed by some wave
  using HT = H16<E>;
  using V8 = typename HT::V8;
  using V4 = typename HT::V4;
  constexpr int NWR = BLK / 32;             // waves per role (32 own rows each)
  constexpr int NW = DUAL ? 2 * NWR : NWR;  // waves of the workgroup
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

  __shared__ __attribute__((aligned(16))) unsigned char X1s[BLK * RB];  // K (dQ) or Q (dK dV)
  __shared__ __attribute__((aligned(16))) unsigned char X2s[BLK * RB];  // V (dQ) or dO (dK dV)
  // dK dV: lse and D of the row block's queries, fetched with its first
  // half (one DMA instruction of wave 0), two blocks' worth by parity
  __shared__ __attribute__((aligned(16))) float Ss[DKDV ? 2 : 1][DKDV ? 256 : 4];

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
  if constexpr (CAUSAL) trim_causal<DKDV>(idx, u, k0, k1);
  const int64_t zh = (int64_t)z * H + h;
  const int64_t Nown = (int64_t)n_own * BLK, Noth = (int64_t)n_oth * BLK;
  const int64_t Nq = DKDV ? Noth : Nown;
  // DUAL: role 0 (the first NWR waves) accumulates dK, role 1 dV
  const int role = DUAL ? wave / NWR : (MODE == MODE_DV ? 1 : 0);
  const int own_lo = u * BLK + (wave % NWR) * 32;  // first own row of this wave

  // ---- the wave's own rows (two tiles) as B fragments: F1 = Q (dQ) or K
  // (dK dV) with the sign of scale*log2(e) folded in (exact), F2 = dO or V
  const float sgn = c > 0.f ? 1.f : (c < 0.f ? -1.f : 0.f);
  const float cs = (c == 0.f) ? 1.f : fabsf(c);
  V8 f1[2][NQ], f2[2][HASDP ? NQ : 1];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const u16* p1 = (DKDV ? K : Q) + (zh * Nown + own_lo + 16 * t + li) * D + 8 * g;
    const u16* p2 = (DKDV ? V : dO) + (zh * Nown + own_lo + 16 * t + li) * D + 8 * g;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      f1[t][q] = *reinterpret_cast<const V8*>(p1 + 32 * q);
      if (HASDP && role == 0) f2[t][q] = *reinterpret_cast<const V8*>(p2 + 32 * q);
      if (sgn != 1.f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f1[t][q][e] = HT::cvt((float)f1[t][q][e] * sgn);
      }
    }
  }
  // dK dV with a key-padding mask: the value of each tile's key (own row)
  float kp_own[2] = {0.f, 0.f};
  if constexpr (KP && DKDV) {
#pragma unroll
    for (int t = 0; t < 2; ++t) kp_own[t] = kpmask[(int64_t)z * Nown + own_lo + 16 * t + li];
  }
  // dQ: the tiles' row statistics: lse2 = lse in log2 units (+inf for a row
  // that saw nothing, so that P = 0 there), D = dO . O, written out as -D
  // (the dK pass starts its dP accumulators from it)
  float lse2_own[2] = {0.f, 0.f}, d_own[2] = {0.f, 0.f};
  if constexpr (!DKDV) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t row = zh * Nq + own_lo + 16 * t + li;
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
  // the other side's matrices and (dK dV) its row statistics for this
  // (batch, head) as raw buffer resources (the launch checks that they fit
  // in 32-bit offsets): each transfer takes a scalar base and offset and a
  // 32-bit per-lane offset
  const __amdgpu_buffer_rsrc_t x1res = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>((DKDV ? Q : K) + zh * Noth * D), 0, (int)(unsigned)(Noth * RB), kRsrcWord3W);
  const __amdgpu_buffer_rsrc_t x2res = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u16*>((DKDV ? dO : V) + zh * Noth * D), 0, (int)(unsigned)(Noth * RB), kRsrcWord3W);
  const __amdgpu_buffer_rsrc_t lres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(lse + zh * Nq), 0, (int)(unsigned)(Nq * 4), kRsrcWord3W);
  const __amdgpu_buffer_rsrc_t dres =
      __builtin_amdgcn_make_buffer_rsrc(Dv + zh * Nq, 0, (int)(unsigned)(Nq * 4), kRsrcWord3W);
  auto dma_half = [&](int o, int x, int par) {
    const unsigned base = (unsigned)(o * BLK + x * HALF) * (unsigned)RB;
    if constexpr (DKDV) {
      if (x == 0 && wave == 0) {
        // lanes 0 .. BLK/4 - 1: 16-byte chunks of lse; the next BLK/4: of D;
        // lanes past those (blocks of 64) repeat D's last chunk into the
        // unused tail of the buffer
        const int ch = lane < BLK / 2 ? lane : BLK / 2 - 1;
        const unsigned qofs = (unsigned)(o * BLK) * 4u;
        if (ch < BLK / 4)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(lres, (lds_u8w*)(&Ss[par][0]), 16, 16u * ch, qofs, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(dres, (lds_u8w*)(&Ss[par][0]), 16, 16u * (ch - BLK / 4), qofs, 0,
                                                   0);
      }
    }
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
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      V8 a[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) a[q] = *reinterpret_cast<const V8*>(xb + 16 * jt * RB + roff[q]);
      __builtin_amdgcn_sched_barrier(0);
      out[0][jt] = init[0][jt];
      out[1][jt] = init[1][jt];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        out[0][jt] = HT::mfma16(a[q], f[0][q], out[0][jt]);
        out[1][jt] = HT::mfma16(a[q], f[1][q], out[1][jt]);
      }
    }
  };
  // acc[t][nt] += X^T (columns 16 nt.., the chunk's 32 rows) . W[t], W the
  // 32 rows of the chunk in the score-register layout (w[t][jt][rr]: row
  // 16 jt + 4 g + rr), rounded to the operand type; both tiles from one
  // pair of transposing reads
  auto tprod = [&](f32x4 (&acc)[2][NNT], const unsigned char* xb, const f32x4 (&w)[2][2]) {
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

  if (k0 < k1) dma_half(idx[k0], 0, 0);
  auto walk = [&](auto mode_c) {
    constexpr int M = decltype(mode_c)::value;
    constexpr bool HDP = M != MODE_DV;
  for (int kk = k0; kk < k1; ++kk) {
    const int o = idx[kk];  // the other side's block
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
      auto issue = [&]() {
        if (x == 0) dma_half(o, 1, 0);
        else if (kk + 1 < k1) dma_half(idx[kk + 1], 0, (kk + 1 - k0) & 1);
      };
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int rofs = x * HALF + 32 * ch;  // first row of the chunk within the block
        const unsigned char* x1 = X1s + rofs * RB;
        const unsigned char* x2 = X2s + rofs * RB;
        f32x4 s[2][2], dp[2][2];
        // dQ with a key-padding mask: the values of the chunk's keys (read
        // while the row products run)
        f32x4 kpv[KP && !DKDV ? 2 : 1];
        if constexpr (KP && !DKDV) {
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
            kpv[jt] = *reinterpret_cast<const f32x4*>(kpmask + (int64_t)z * Noth + o * BLK + rofs + 16 * jt + 4 * g);
        }
        // element (own row 16 t + li, other row rofs + 16 jt + 4 g + rr);
        // dK dV: the chunk's lse and -D (read while the row products run)
        f32x4 l4[2], d4[2];
        if constexpr (DKDV) {
          const float* st = &Ss[(kk - k0) & 1][0];
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            l4[jt] = *reinterpret_cast<const f32x4*>(st + rofs + 16 * jt + 4 * g);
            if constexpr (HDP) d4[jt] = *reinterpret_cast<const f32x4*>(st + BLK + rofs + 16 * jt + 4 * g);
          }
        }
        // S starts from 0, dP from -D: the product then holds dP - D
        const f32x4 zero[2][2] = {};
        f32x4 nd[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) {
            if constexpr (DKDV) nd[t][jt] = d4[jt];
            else nd[t][jt] = f32x4{-d_own[t], -d_own[t], -d_own[t], -d_own[t]};
          }
        rprod(s, x1, f1, zero);
        if constexpr (HDP) rprod(dp, x2, f2, nd);
        if (ch == 0) issue();
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              float xv = s[t][jt][rr] * cs;
              if constexpr (KP) xv = fmaf(DKDV ? kp_own[t] : kpv[jt][rr], kLog2eW, xv);
              float l2;
              if constexpr (DKDV) {
                // a row with nothing visible (lse = -inf: P = 0 there) needs
                // a key-padding mask: without one every query row of a
                // visited block sees keys of it (causal: its diagonal key)
                const float l = l4[jt][rr];
                l2 = (KP && l == -INFINITY) ? INFINITY : l * kLog2eW;
              } else {
                l2 = lse2_own[t];
              }
              if (CAUSAL && mask_block) {
                const int own_r = own_lo + 16 * t + li, oth = o * BLK + rofs + 16 * jt + 4 * g + rr;
                if (DKDV ? (own_r > oth) : (oth > own_r)) xv = -INFINITY;
              }
              const float p = __builtin_amdgcn_exp2f(xv - l2);
              s[t][jt][rr] = p;
              if constexpr (HDP) dp[t][jt][rr] *= p;  // (dP - D) P = dS / scale
            }
        if constexpr (M == MODE_DV) tprod(acc, x2, s);  // dV^T += dO^T P
        else tprod(acc, x1, dp);  // dQ^T += K^T dS^T, dK^T += Q^T dS
      }
    }
  }
  };
  // the whole walk for a wave of mode M: the kernel's mode, or with DUAL
  // the wave's role (both roles meet at the same barriers)
  if constexpr (DUAL) {
    if (role == 0) walk(std::integral_constant<int, MODE_DK>{});
    else walk(std::integral_constant<int, MODE_DV>{});
  } else {
    walk(std::integral_constant<int, MODE>{});
  }

  // ---- results: lane (g, li) holds columns 16 nt + 4 g .. of own row 16 t + li;
  // dQ and dK take the scale of dS here, once per element
  const float osc = (DUAL ? role == 0 : MODE != MODE_DV) ? scale : 1.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    u16* pg = (DUAL && role == 1 ? G2 : G) + (zh * Nown + own_lo + 16 * t + li) * D + 4 * g;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt)
      *reinterpret_cast<V4*>(pg + nt * 16) = V4{HT::cvt(acc[t][nt][0] * osc), HT::cvt(acc[t][nt][1] * osc),
                                                HT::cvt(acc[t][nt][2] * osc), HT::cvt(acc[t][nt][3] * osc)};
  }
}

template <typename E, int BLK, int D, int MODE>
int launch_w(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  const bool kp = a.kp != nullptr;
  constexpr bool DKDV = MODE != MODE_DQ;
  const int n_own = DKDV ? L->nbc : L->nbr, n_oth = DKDV ? L->nbr : L->nbc;
  const dim3 grid(L->H * n_own * a.Z), block(BLK * 2 * (MODE == MODE_DKV ? 2 : 1));
  const int32_t* ptr = DKDV ? L->col_ptr : L->row_ptr;
  const int32_t* idx = DKDV ? L->row_idx : L->col_idx;
  const int32_t* order = DKDV ? L->col_order : L->row_order;
  const int32_t* order_h = DKDV ? L->col_order_h : L->row_order_h;
  // head-grouped XCD order with rows (columns) of similar length, as the
  // 16-row kernels (two workgroups per CU)
  const double per_slot = (double)a.Z * (double)L->nnz / (2.0 * L->num_cus);
  const int max_len = DKDV ? L->max_col_len : L->max_row_len;
  const int grouped = (4.0 * max_len <= per_slot) ? 1 : 0;
  const float c = a.scale * kLog2eW;
  u16* g = (u16*)(MODE == MODE_DQ ? a.dQ : (MODE == MODE_DV ? a.dV : a.dK));
#define BSA_BWDW_LAUNCH(CA, KPM)                                                                                 \
  hipLaunchKernelGGL((k_bwd_wide<E, BLK, D, CA, MODE, KPM>), grid, block, 0, s, ptr, idx, order, order_h,        \
                     grouped, (const u16*)a.Q, (const u16*)a.K, (const u16*)a.V, (const u16*)a.O, (const u16*)a.dO, \
                     g, a.lse, a.Dws, a.Z, L->H, n_own, n_oth, c, a.scale, a.kp, (u16*)a.dV)
  if (a.causal) {
    if (kp) BSA_BWDW_LAUNCH(true, true);
    else BSA_BWDW_LAUNCH(true, false);
  } else {
    if (kp) BSA_BWDW_LAUNCH(false, true);
    else BSA_BWDW_LAUNCH(false, false);
  }
#undef BSA_BWDW_LAUNCH
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

template <typename E, int BLK, int D>
int run_w(const bs_layout* L, const BwdArgs& a, hipStream_t s) {
  if (int rc = launch_w<E, BLK, D, MODE_DQ>(L, a, s)) return rc;  // dQ and D
  return launch_w<E, BLK, D, MODE_DKV>(L, a, s);                  // dK and dV (reads D)
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
