// Fused attention on slope-1 ACSR layouts with each K/V block staged once for
// several block rows (float32 operands).
//
// On such a layout (SPLAT abstract: the affine-compressed sparse row format
// and the just-in-time analysis of a pattern's regular geometry), block row r
// holds the columns r + o for o in one sorted offset set O, clipped to the
// grid. Rows r and r + t share every column r + t + o for which o + t is in O
// as well: a strided term shifted by a multiple of its stride maps onto
// itself, and a window shifted by t keeps all but t of its blocks. The host
// (api.cpp) picks the row stride t with the largest overlap and groups G
// rows r0, r0 + t, ..., r0 + (G-1) t into one workgroup. The group's columns
// are r0 + u for u in the union U of O, O + t, ..., O + (G-1) t; next to each
// u, a bit mask of the rows that hold it. The workgroup walks U in ascending
// order and stages each block's K and V into LDS once, and the waves of every
// row that holds the block compute on it; a row sees its own blocks in
// ascending column order, as the one-row-per-workgroup kernel does, with the
// same per-block arithmetic (scores on 16x16x4 float32 MFMA, the streaming
// softmax with lazy rescale, P.V straight from the score registers).
//
// G = 2 rows (four waves at blocks of 32, eight at 64). A step: barrier
// (every wave is done with the block in LDS), store the next block from
// registers, barrier, load the block after it into registers (in flight
// during the compute), compute. Measured on strided_acsr_b32 (one process,
// interleaved, medians of 21): this kernel 389 us, the one-row kernel 391;
// four rows per workgroup 408 (409 with double-buffered LDS); two rows with
// double-buffered LDS 399. The fp32 kernel is bound by the matrix cores and
// the softmax between them, not by staging (16 flops per staged byte), so
// staging a block once for two rows saves little.
#include <math.h>

#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

constexpr float kLog2eB = 1.4426950408889634f;
constexpr float kLn2B = 0.6931471805599453f;
constexpr float kTauB = 8.0f;  // lazy-rescale headroom, log2 units

// uoff, umask: the union offsets (ascending) and their row masks, nu entries;
// grp: the first row r0 of every group, longest group first; grid: groups x
// Z x H, the batch index fastest. Q, K, V, O: [Z][H][N][D] float32.
template <int BLK, int D, int G, bool CAUSAL>
__global__ __launch_bounds__(G * BLK * 4) void k_attn_band(
    const int32_t* __restrict__ uoff, const int32_t* __restrict__ umask, int nu, const int32_t* __restrict__ grp,
    int stride, const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, int Z, int H, int nbr, int nbc, float c, float* __restrict__ lse) {
  constexpr int NW = BLK / 16;      // waves per block row
  constexpr int NT = 64 * NW * G;   // threads
  constexpr int NQ = D / 16;        // Q fragments (4 floats) per lane
  constexpr int NJT = BLK / 16;     // 16-key tiles per block
  constexpr int NNT = D / 16;       // 16-column tiles of O
  constexpr int KSTR = D + 8;       // padded LDS rows, as in the one-row kernel (conflict-free reads)
  constexpr int VSTR = D + 4;
  constexpr int KBUF = BLK * KSTR, VBUF = BLK * VSTR, STAGE = KBUF + VBUF;
  constexpr int CPR = D / 4;             // 16-byte chunks per row
  constexpr int KCH = BLK * CPR / NT;    // chunks per thread and matrix
  static_assert(KCH >= 1 && BLK * CPR % NT == 0, "staging");
  __shared__ __attribute__((aligned(16))) float lds[STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = w / NW, wr = w % NW;  // row of the group, query tile of the row
  const int li = lane & 15, g = lane >> 4;
  const int zhn = Z * H;
  const int r0 = grp[blockIdx.x / zhn];
  const int z = (blockIdx.x % zhn) % Z, h = (blockIdx.x % zhn) / Z;
  const int r = r0 + j * stride;
  const bool row_ok = r < nbr;
  int vm = 0;  // rows of the group that are on the grid
#pragma unroll
  for (int t = 0; t < G; ++t)
    if (r0 + t * stride < nbr) vm |= 1 << t;
  // the group's columns r0 + uoff[i], i in [i_lo, i_hi)
  auto first_at_least = [&](int v) {
    int lo = 0, hi = nu;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (uoff[mid] < v) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  const int i_lo = first_at_least(-r0), i_hi = first_at_least(nbc - r0);
  auto advance = [&](int i) {  // next entry held by a row on the grid
    while (i < i_hi && (umask[i] & vm) == 0) ++i;
    return i;
  };

  const int64_t zh = (int64_t)z * H + h;
  const int64_t Nq = (int64_t)nbr * BLK, Nk = (int64_t)nbc * BLK;
  const int q_lo = r * BLK + wr * 16;
  const int q_index = q_lo + li;
  const float* Kz = K + zh * Nk * D;
  const float* Vz = V + zh * Nk * D;

  // Q as B fragments with scale*log2(e) folded in
  f32x4 qf[NQ];
  {
    const float* pq = Q + (zh * Nq + (row_ok ? q_index : li)) * D + g * 4;
#pragma unroll
    for (int u = 0; u < NQ; ++u) qf[u] = *reinterpret_cast<const f32x4*>(pq + u * 16) * c;
  }

  int goff[KCH], koff[KCH], voff[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int ch = tid + i * NT;
    goff[i] = (ch / CPR) * D + (ch % CPR) * 4;
    koff[i] = (ch / CPR) * KSTR + (ch % CPR) * 4;
    voff[i] = (ch / CPR) * VSTR + (ch % CPR) * 4;
  }
  f32x4 rk[KCH], rv[KCH];
  auto load = [&](int cb) {
    const int64_t base = (int64_t)cb * BLK * D;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      rk[i] = *reinterpret_cast<const f32x4*>(Kz + base + goff[i]);
      rv[i] = *reinterpret_cast<const f32x4*>(Vz + base + goff[i]);
    }
  };
  auto store = [&](float* dst) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      *reinterpret_cast<f32x4*>(dst + koff[i]) = rk[i];
      *reinterpret_cast<f32x4*>(dst + KBUF + voff[i]) = rv[i];
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[NNT];
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int i = advance(i_lo);
  if (i < i_hi) load(r0 + uoff[i]);
  while (i < i_hi) {
    const int inext = advance(i + 1);
    __syncthreads();
    store(lds);
    __syncthreads();
    if (inext < i_hi) load(r0 + uoff[inext]);
    const int cb = r0 + uoff[i];
    const bool mine = row_ok && ((umask[i] >> j) & 1);
    // blocks whose every key is after every query of this wave add nothing
    const bool compute = mine && !(CAUSAL && cb * BLK > q_lo + 15);
    const bool mask_block = CAUSAL && (cb * BLK + BLK - 1 > q_lo);
    const float* Kb = lds;
    const float* Vb = Kb + KBUF;
    if (compute) {
      // ---- S^T = K Q^T: s[jt][rr] = score of (query li, key 16 jt + 4 g + rr)
      f32x4 s[NJT];
      const float* kbase = &Kb[li * KSTR + g * 4];
      f32x4 ka[2][NQ];
#pragma unroll
      for (int u = 0; u < NQ; ++u) ka[0][u] = *reinterpret_cast<const f32x4*>(kbase + u * 16);
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        if (jt + 1 < NJT) {
#pragma unroll
          for (int u = 0; u < NQ; ++u)
            ka[(jt + 1) & 1][u] = *reinterpret_cast<const f32x4*>(kbase + 16 * (jt + 1) * KSTR + u * 16);
        }
        s[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NQ; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[jt & 1][u][e], qf[u][e], s[jt], 0, 0, 0);
      }
      // ---- causal mask, block max, lazy rescale, exp2
      if (mask_block) {
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            if (cb * BLK + 16 * jt + 4 * g + rr > q_index) s[jt][rr] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, s[jt][rr]);
      mx = rows4_max(mx);
      const bool upd = mx > m_run + kTauB;
      if (__builtin_amdgcn_ballot_w64(upd) != 0) {
        // a row that has seen nothing (m_run = -inf) keeps l = 0 and O = 0
        // through alpha = 0; rows without an update keep their sums
        const float m_new = upd ? mx : m_run;
        const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) o[nt] *= alpha;
        m_run = m_new;
      }
      const float m_sub = (m_run == -INFINITY) ? 0.f : m_run;
      float ls = 0.f;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          s[jt][rr] = __builtin_amdgcn_exp2f(s[jt][rr] - m_sub);
          ls += s[jt][rr];
        }
      l_run += ls;
      // ---- O^T += V^T P^T, one V element per lane and instruction; tile
      // jt+1 read while tile jt is multiplied
      float va[2][4][NNT];
      const float* vbase = &Vb[(4 * g) * VSTR + li];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) va[0][rr][nt] = vbase[rr * VSTR + nt * 16];
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        if (jt + 1 < NJT) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) va[(jt + 1) & 1][rr][nt] = vbase[(16 * (jt + 1) + rr) * VSTR + nt * 16];
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int nt = 0; nt < NNT; ++nt)
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[jt & 1][rr][nt], s[jt][rr], o[nt], 0, 0, 0);
      }
    }
    i = inext;
  }

  if (!row_ok) return;
  l_run = rows4_sum(l_run);
  const float inv = (l_run > 0.f) ? 1.0f / l_run : 0.f;
  // natural-log log-sum-exp of the row: l sums exp2(x - m_run), x in log2 units
  if (lse != nullptr && g == 0)
    lse[zh * Nq + q_index] = (l_run > 0.f) ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2B : -INFINITY;
  float* po = O + (zh * Nq + q_index) * D + 4 * g;
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) *reinterpret_cast<f32x4*>(po + nt * 16) = o[nt] * inv;
}

template <int BLK, int D>
int launch_bd(const bs_layout* L, const AttnArgs& a, hipStream_t s) {
  constexpr int G = 2;
  const dim3 grid((unsigned)((int64_t)L->share_ngrp * a.Z * L->H)), block(G * BLK * 4);
  const float c = a.scale * kLog2eB;
  if (a.causal)
    hipLaunchKernelGGL((k_attn_band<BLK, D, G, true>), grid, block, 0, s, L->share_uoff, L->share_umask, L->share_n,
                       L->share_grp, L->share_stride, (const float*)a.Q, (const float*)a.K, (const float*)a.V,
                       (float*)a.O, a.Z, L->H, L->nbr, L->nbc, c, a.lse);
  else
    hipLaunchKernelGGL((k_attn_band<BLK, D, G, false>), grid, block, 0, s, L->share_uoff, L->share_umask, L->share_n,
                       L->share_grp, L->share_stride, (const float*)a.Q, (const float*)a.K, (const float*)a.V,
                       (float*)a.O, a.Z, L->H, L->nbr, L->nbc, c, a.lse);
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

}  // namespace

int launch_attention_band(const bs_layout* L, const AttnArgs& a, hipStream_t s) {
  // float32: only on request (it measured the same time as the one-row
  // kernel on strided_acsr_b32)
  if (L->share_mode != 1 || L->share_n == 0 || a.dt != BS_F32 || a.am != nullptr || a.kp != nullptr)
    return kNotApplicable;
  if (L->share_rows != 2) return kNotApplicable;
  if (L->block == 32) return a.d == 64 ? launch_bd<32, 64>(L, a, s) : launch_bd<32, 128>(L, a, s);
  if (L->block == 64 && a.d == 64) return launch_bd<64, 64>(L, a, s);
  return kNotApplicable;
}

}  // namespace bsa
