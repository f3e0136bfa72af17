// Fused block-sparse attention: SDD -> block-sparse softmax -> DSD in one
// kernel (the composition of Triton issue 117, "question on blocksparse"),
// with the streaming softmax of the Triton tutorial (Puzzle 8, online
// softmax; Puzzle 9, simple FlashAttention): a running row max m and sum l,
// the partial output rescaled by exp(m_old - m_new) when the reference max
// moves, and one division by l at the end (the same value as normalising at
// every step).
//
// Work decomposition. One workgroup per (batch, head, block row), rows
// taken longest first; b/16 waves, wave w owning query rows 16w..16w+15 of
// the block. The stored blocks of the row are visited in order; each is
// staged once into LDS for all waves, K and V both row-major (contiguous
// 16-byte writes), and the next block is already in flight into registers
// while the current one is computed. Row strides were chosen by measuring
// the operand read patterns on gfx950: K rows padded to 32 mod 256 bytes,
// fp32 V rows to 16 mod 64 bytes, bf16 V rows to 32 mod 256 bytes; every
// operand read below is then free of bank conflicts.
//
// Per block and wave, with 16x16 MFMA tiles (fp32 16x16x4, bf16 16x16x32):
//   S^T = K_c Q^T     A = K rows from LDS, B = the wave's Q rows (registers,
//                     loaded once). In the accumulator every lane then owns
//                     ONE query row (its column) and 4 keys per 16-key tile,
//                     so row max / sum are in-lane plus one butterfly over
//                     the 4 lane groups.
//   softmax           log2 domain (scale*log2(e) folded into Q for fp32, into
//                     one fma for bf16); causal mask only on blocks that
//                     reach the diagonal; raw v_exp_f32. The reference max
//                     moves only when a block's max exceeds it by more than
//                     TAU (so p <= 2^TAU): numerator and denominator share it,
//                     so the result is exact, and most blocks skip the
//                     rescale of O.
//   O^T += V_c^T P^T  A = V^T, B = P^T straight from the score registers (no
//                     transpose); O^T also keeps one query row per lane, so
//                     the rescale is a per-lane scalar. fp32 takes one V
//                     element per lane and instruction (one 4-byte LDS read);
//                     bf16 takes 8 keys of one column per lane from two
//                     ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x
//                     16-column patch and every lane receives the 4 keys of
//                     its own column), so V never needs a transposed copy.
// bf16: P is rounded to bf16 (RNE) for P.V, O once at the end.
#include <math.h>

#include <type_traits>

#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTau = 8.0f;  // lazy-rescale headroom, log2 units

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename E>
struct Cfg;
template <>
struct Cfg<float> {
  static constexpr int VEC = 4;   // elements per 16-byte vector
  static constexpr int KC = 16;   // contraction values per 16-byte lane vector group (4 groups x 4)
  typedef f32x4 Vec;
};
template <>
struct Cfg<bf16_t> {
  static constexpr int VEC = 8;
  static constexpr int KC = 32;
  typedef bf16x8 Vec;
};

// padded LDS row strides (elements), measured free of bank conflicts for the
// operand reads of the kernel: K rows 32 mod 256 bytes; V rows 16 mod 64
// bytes (fp32, one 4-byte read per lane) or 32 mod 256 bytes (bf16,
// transposing 8-byte reads)
template <typename E, int BLK, int D>
struct Lds {
  using St = typename Elem<E>::storage;
  static constexpr int KSTR = D + 32 / (int)sizeof(St);
  static constexpr int VSTR = std::is_same<E, bf16_t>::value ? D + 16 : D + 4;
  static constexpr size_t STAGE = (size_t)BLK * (KSTR + VSTR) * sizeof(St);  // bytes per key group
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 4 keys of one V column per lane, from a row-major bf16 tile in LDS: the
// 16 lanes of a group pass the addresses of a 4-row x 16-column patch (lane
// 4k + m: row k, columns 4m..4m+3) and lane i receives column i of the 4 rows
__device__ __forceinline__ bf16x4 lds_read_tr16(const u16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)((__attribute__((address_space(3))) u16*)p));
  return __builtin_bit_cast(bf16x4, v);
}

template <typename E, int BLK, int D, bool CAUSAL, int NS>
__global__ __launch_bounds__(BLK * 4 * NS) void k_attn(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, const int32_t* __restrict__ row_order,
    const typename Elem<E>::storage* __restrict__ Q, const typename Elem<E>::storage* __restrict__ K,
    const typename Elem<E>::storage* __restrict__ V, typename Elem<E>::storage* __restrict__ O, int Z, int H,
    int nbr, int nbc, float c) {
  using St = typename Elem<E>::storage;
  using Vec = typename Cfg<E>::Vec;
  constexpr bool BF = std::is_same<E, bf16_t>::value;
  constexpr int VEC = Cfg<E>::VEC, KC = Cfg<E>::KC;
  constexpr int NW = BLK / 16, NT = 64 * NW;  // waves / threads of one key group
  constexpr int NQ = D / KC;          // Q fragments per lane
  // Staging of the next block: split (K during the score product, V during
  // softmax and P.V, one matrix in registers at a time) where registers are
  // the limit, else both at the start of a step, hidden by the whole step.
  constexpr bool SPLIT = BF && D == 128;
  constexpr int KS = BLK < 64 ? BLK : 64;  // keys per softmax sub-step
  constexpr int NSUB = BLK / KS;
  constexpr int NJT = KS / 16;        // 16-key tiles per sub-step
  constexpr int NNT = D / 16;         // 16-column tiles of O
  constexpr int KSTR = Lds<E, BLK, D>::KSTR;
  constexpr int VSTR = Lds<E, BLK, D>::VSTR;
  constexpr int CPR = D / VEC;        // 16-byte chunks per row
  constexpr int KCH = BLK * CPR / NT; // chunks per thread and matrix (D / (4 VEC))
  static_assert(KCH >= 1 && BLK * CPR % NT == 0, "staging");

  constexpr int KBUF = BLK * KSTR, VBUF = BLK * VSTR;  // one stage of one key group
  constexpr int MERGE = NS > 1 ? (NS - 1) * NW * 64 * (2 + 4 * NNT) : 0;  // floats for the final merge
  static_assert((size_t)MERGE * 4 <= (size_t)NS * (KBUF + VBUF) * sizeof(St), "merge area");

  __shared__ __attribute__((aligned(16))) St Ks[NS * KBUF];
  __shared__ __attribute__((aligned(16))) St Vs[NS * VBUF];

  const int tid_all = threadIdx.x;
  const int sg = __builtin_amdgcn_readfirstlane(tid_all / NT);  // key group of this wave
  const int tid = tid_all % NT;                                 // thread index inside the key group
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // query tile; uniform keeps mask tests scalar
  const int lane = tid & 63;
  St* const Kg = Ks + sg * KBUF;
  St* const Vg = Vs + sg * VBUF;
  const int li = lane & 15, g = lane >> 4;
  // 1-D grid, batch fastest: dispatch follows the longest-first order
  // across the whole batch
  const int hr = row_order[blockIdx.x / Z];
  const int z = blockIdx.x % Z;
  const int h = hr / nbr, r = hr % nbr;
  const int k0 = row_ptr[hr], k1 = row_ptr[hr + 1];
  const int64_t zh = (int64_t)z * H + h;
  const int64_t Nq = (int64_t)nbr * BLK, Nk = (int64_t)nbc * BLK;
  const int q_lo = r * BLK + wave * 16;  // first query row of this wave
  const int q_index = q_lo + li;         // this lane's query row
  const St* Kz = K + zh * Nk * D;
  const St* Vz = V + zh * Nk * D;

  // ---- Q as B fragments; fp32 folds scale*log2(e) in, bf16 only its sign
  Vec qf[NQ];
  float cs;
  {
    const St* pq = Q + (zh * Nq + q_index) * D + g * VEC;
#pragma unroll
    for (int u = 0; u < NQ; ++u) qf[u] = *reinterpret_cast<const Vec*>(pq + u * KC);
    if constexpr (BF) {
      const float sgn = c > 0.f ? 1.f : (c < 0.f ? -1.f : 0.f);
      if (sgn != 1.f) {
#pragma unroll
        for (int u = 0; u < NQ; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[u][e] = to_bf16((float)qf[u][e] * sgn);  // exact
      }
      cs = (c == 0.f) ? 1.f : fabsf(c);
    } else {
#pragma unroll
      for (int u = 0; u < NQ; ++u) qf[u] *= c;
      cs = 1.f;
    }
  }

  // ---- staging of one block: K and V use the same chunk mapping; with
  // SPLIT they share registers (held at different times)
  Vec stg[KCH];
  Vec stv[SPLIT ? 1 : KCH];
  // per-thread chunk offsets (elements) into a global block and into the
  // padded LDS rows, computed once
  int goff[KCH], koff[KCH], voff[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int ch = tid + i * NT;
    goff[i] = (ch / CPR) * D + (ch % CPR) * VEC;
    koff[i] = (ch / CPR) * KSTR + (ch % CPR) * VEC;
    voff[i] = (ch / CPR) * VSTR + (ch % CPR) * VEC;
  }
  auto stage_load_to = [&](Vec* r, const St* base, int cb) {
    const St* src = base + (int64_t)cb * BLK * D;  // uniform
#pragma unroll
    for (int i = 0; i < KCH; ++i) r[i] = *reinterpret_cast<const Vec*>(src + goff[i]);
  };
  auto stage_store_from = [&](const Vec* r, St* dst, const int* off) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) *reinterpret_cast<Vec*>(&dst[off[i]]) = r[i];
  };
  auto stage_load = [&](const St* base, int cb) { stage_load_to(stg, base, cb); };
  auto stage_store = [&](St* dst, const int* off) { stage_store_from(stg, dst, off); };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[NNT];
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // key group sg takes blocks k0 + sg, k0 + sg + NS, ... of the row.
  // Without SPLIT a step is: barrier, store K and V of this block, barrier,
  // load K and V of the next block (in flight during the compute), compute.
  // With SPLIT: K of the next block is loaded during the score product and
  // stored once every wave is past it; V of the next block is loaded then
  // and stored once every wave is past P.V.
  const int nsteps = (k1 - k0 + NS - 1) / NS;
  if (k0 + sg < k1) {
    stage_load(Kz, col_idx[k0 + sg]);
    if constexpr (SPLIT) {
      stage_store(Kg, koff);
      stage_load(Vz, col_idx[k0 + sg]);
      stage_store(Vg, voff);
    } else {
      stage_load_to(stv, Vz, col_idx[k0 + sg]);
    }
  }
  if constexpr (SPLIT) __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const int kk = k0 + step * NS + sg;
    const bool valid = kk < k1;
    const bool has_next = kk + NS < k1;
    const int cb_next = has_next ? col_idx[kk + NS] : 0;
    if constexpr (!SPLIT) {
      __syncthreads();  // every wave is done with the previous blocks in LDS
      if (valid) {
        stage_store(Kg, koff);
        stage_store_from(stv, Vg, voff);
      }
      __syncthreads();
      if (has_next) {
        stage_load(Kz, cb_next);
        stage_load_to(stv, Vz, cb_next);
      }
    } else {
      if (has_next) stage_load(Kz, cb_next);
    }
    const int cb = valid ? col_idx[kk] : 0;
    // blocks whose every key is after every query of this wave add nothing
    const bool compute = valid && !(CAUSAL && cb * BLK > q_lo + 15);
    const bool mask_block = CAUSAL && (cb * BLK + BLK - 1 > q_lo);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
    const int kofs = sub * KS;  // first key of this sub-step within the block

    // S^T tiles: s[jt][rr] = score(query li, key kofs + 16 jt + 4 g + rr). The K
    // operands of tile jt+1 are read from LDS while tile jt is multiplied.
    f32x4 s[NJT];
    const St* kbase = &Kg[(kofs + li) * KSTR + g * VEC];
    if (!compute) {
    } else if constexpr (BF) {
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        s[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
          const Vec a = *reinterpret_cast<const Vec*>(kbase + 16 * jt * KSTR + u * KC);
          s[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[u], s[jt], 0, 0, 0);
        }
      }
    } else {
      Vec ka[2][NQ];
#pragma unroll
      for (int u = 0; u < NQ; ++u) ka[0][u] = *reinterpret_cast<const Vec*>(kbase + u * KC);
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        if (jt + 1 < NJT) {
#pragma unroll
          for (int u = 0; u < NQ; ++u)
            ka[(jt + 1) & 1][u] = *reinterpret_cast<const Vec*>(kbase + 16 * (jt + 1) * KSTR + u * KC);
        }
        s[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NQ; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[jt & 1][u][e], qf[u][e], s[jt], 0, 0, 0);
      }
    }

    if (SPLIT && sub == NSUB - 1) {
      __syncthreads();  // every wave is past the score product: K of the next block may land
      if (has_next) {
        stage_store(Kg, koff);
        stage_load(Vz, cb_next);
      }
    }
    if (compute) {
    // mask and block max (raw scores; cs > 0)
    if (mask_block) {
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (cb * BLK + kofs + 16 * jt + 4 * g + rr > q_index) s[jt][rr] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, s[jt][rr]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_blk = mx * cs;
    const bool upd = m_blk > m_run + kTau;
    if (__builtin_amdgcn_ballot_w64(upd) != 0) {  // wave-uniform
      const float m_new = upd ? m_blk : m_run;
      const float alpha = fast_exp2(m_run - m_new);  // 0 when m_run = -inf
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
        const float p = fast_exp2(fmaf(s[jt][rr], cs, -m_sub));
        s[jt][rr] = p;
        ls += p;
      }
    l_run += ls;

    // O^T[n][query] += V^T[n][keys] P^T[keys][query]
    if constexpr (BF) {
      // lane (g, j = 4k + m) points at row 16h + 4g + k, columns 4m.. of
      // the n-tile; it gets back keys 16h + 4g + 0..3 of column nt*16 + li
      const u16* vb = &Vg[(kofs + 4 * g + (li >> 2)) * VSTR + 4 * (li & 3)];
      if constexpr (NJT >= 2) {
        // operands read right before use: the bf16 kernel is register bound
        // (two 8-wave workgroups per CU need <= 128 VGPRs)
#pragma unroll
        for (int jp = 0; jp < NJT / 2; ++jp) {
          const bf16x8 pb = {to_bf16(s[2 * jp][0]),     to_bf16(s[2 * jp][1]),     to_bf16(s[2 * jp][2]),
                             to_bf16(s[2 * jp][3]),     to_bf16(s[2 * jp + 1][0]), to_bf16(s[2 * jp + 1][1]),
                             to_bf16(s[2 * jp + 1][2]), to_bf16(s[2 * jp + 1][3])};
#pragma unroll
          for (int nt = 0; nt < NNT; ++nt) {
            const bf16x4 a0 = lds_read_tr16(vb + (32 * jp) * VSTR + nt * 16);
            const bf16x4 a1 = lds_read_tr16(vb + (32 * jp + 16) * VSTR + nt * 16);
            const bf16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[nt], 0, 0, 0);
          }
        }
      } else {  // a single 16-key tile: the other half of the k range is zero
        const __bf16 zb = (__bf16)0.f;
        const bf16x8 pb = {to_bf16(s[0][0]), to_bf16(s[0][1]), to_bf16(s[0][2]), to_bf16(s[0][3]), zb, zb, zb, zb};
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) {
          const bf16x4 a0 = lds_read_tr16(vb + nt * 16);
          const bf16x8 a = {a0[0], a0[1], a0[2], a0[3], zb, zb, zb, zb};
          o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[nt], 0, 0, 0);
        }
      }
    } else {
      // one V element per lane and instruction; tile jt+1 is read while
      // tile jt is multiplied
      float va[2][4][NNT];
      const float* vbase = &Vg[(kofs + 4 * g) * VSTR + li];
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
    }  // compute
    }  // sub-step
    if constexpr (SPLIT) {
      __syncthreads();  // every wave is past P.V: V of the next block may land
      if (has_next) stage_store(Vg, voff);
      // with sub-steps, the first P.V of the next block precedes its
      // mid-block barrier, so V must be visible before the next step starts
      if constexpr (NSUB > 1) __syncthreads();
    }
  }

  // ---- merge the key groups: (m, l, O) of group sg > 0 through LDS into
  // group 0, rescaling each side by exp2(m_side - m_max)
  if constexpr (NS > 1) {
    constexpr int SLOT = 64 * (2 + 4 * NNT);
    float* red = reinterpret_cast<float*>(Ks);
    __syncthreads();
    if (sg > 0) {
      float* slot = red + ((sg - 1) * NW + wave) * SLOT;
      slot[lane] = m_run;
      slot[64 + lane] = l_run;
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) slot[128 + (nt * 4 + e) * 64 + lane] = o[nt][e];
    }
    __syncthreads();
    if (sg > 0) return;
#pragma unroll
    for (int s2 = 1; s2 < NS; ++s2) {
      const float* slot = red + ((s2 - 1) * NW + wave) * SLOT;
      const float m2 = slot[lane], l2 = slot[64 + lane];
      const float m_new = fmaxf(m_run, m2);
      const float a1 = (m_new == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      const float a2 = (m_new == -INFINITY) ? 0.f : fast_exp2(m2 - m_new);
      l_run = l_run * a1 + l2 * a2;
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[nt][e] = o[nt][e] * a1 + slot[128 + (nt * 4 + e) * 64 + lane] * a2;
      m_run = m_new;
    }
  }

  // ---- finish: l over the 4 lane groups, O = O^T / l, 4 columns per store
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  const float inv = (l_run > 0.f) ? 1.0f / l_run : 0.f;
  St* po = O + (zh * Nq + q_index) * D + 4 * g;
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) {
    if constexpr (BF) {
      *reinterpret_cast<bf16x4*>(po + nt * 16) =
          bf16x4{to_bf16(o[nt][0] * inv), to_bf16(o[nt][1] * inv), to_bf16(o[nt][2] * inv), to_bf16(o[nt][3] * inv)};
    } else {
      *reinterpret_cast<f32x4*>(po + nt * 16) = o[nt] * inv;
    }
  }
}

template <typename E, int BLK, int D, int NS>
int launch_ns(const bs_layout* L, const void* Q, const void* K, const void* V, void* O, int Z, float c, bool causal,
              hipStream_t s) {
  using St = typename Elem<E>::storage;
  const dim3 grid(L->H * L->nbr * Z), block(BLK * 4 * NS);
  if (causal)
    hipLaunchKernelGGL((k_attn<E, BLK, D, true, NS>), grid, block, 0, s, L->row_ptr, L->col_idx, L->row_order,
                       (const St*)Q, (const St*)K, (const St*)V, (St*)O, Z, L->H, L->nbr, L->nbc, c);
  else
    hipLaunchKernelGGL((k_attn<E, BLK, D, false, NS>), grid, block, 0, s, L->row_ptr, L->col_idx, L->row_order,
                       (const St*)Q, (const St*)K, (const St*)V, (St*)O, Z, L->H, L->nbr, L->nbc, c);
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

// Key groups per workgroup. With one group, about four workgroups share a
// CU, so a row of n blocks needs ~4n block-times of its CU while the CU's
// whole share of the job is Z*nnz/CUs block-times: once the longest row
// exceeds that, it sets the end of the kernel. NS groups cut the row's own
// time by NS (the groups run its blocks side by side and merge at the end).
inline int pick_key_groups(const bs_layout* L, int Z, int max_ns) {
  const double per_cu = (double)Z * (double)L->nnz / L->num_cus;
  int ns = 1;
  while (ns < max_ns && 4.0 * L->max_row_len / ns > per_cu) ns *= 2;
  return ns;
}

template <typename E, int BLK, int D>
int run(const bs_layout* L, const void* Q, const void* K, const void* V, void* O, int Z, float c, bool causal,
        hipStream_t s) {
  // largest key-group count (up to 4, and 1024 threads) whose LDS fits in 160 KiB
  constexpr size_t stage = Lds<E, BLK, D>::STAGE;
  constexpr int max_ns = (BLK <= 64 && 4 * stage <= 160 * 1024) ? 4 : ((BLK <= 64 && 2 * stage <= 160 * 1024) ? 2 : 1);
  const int ns = pick_key_groups(L, Z, max_ns);
  if constexpr (max_ns >= 4) {
    if (ns >= 4) return launch_ns<E, BLK, D, 4>(L, Q, K, V, O, Z, c, causal, s);
  }
  if constexpr (max_ns >= 2) {
    if (ns >= 2) return launch_ns<E, BLK, D, 2>(L, Q, K, V, O, Z, c, causal, s);
  }
  return launch_ns<E, BLK, D, 1>(L, Q, K, V, O, Z, c, causal, s);
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
