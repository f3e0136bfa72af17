// The row-block kernel (template) and its launch machinery, shared by the
// translation units that instantiate its modes (attention.hip: fused
// attention, SDD, DSD, DSD^T; attention_masked.hip: fused attention with
// dense masks).
//
// Fused block-sparse attention: SDD -> block-sparse softmax -> DSD in one
// kernel (the composition of Triton issue 117, "question on blocksparse"),
// with the streaming softmax of the Triton tutorial (Puzzle 8, online
// softmax; Puzzle 9, simple FlashAttention): a running row max m and sum l,
// the partial output rescaled by exp(m_old - m_new) when the reference max
// moves, and one division by l at the end (the same value as normalising at
// every step). The same kernel, with the softmax and one of the two products
// compiled out, is the SDD (scores written out) and the DSD (P read in).
//
// Work decomposition. One workgroup per (batch, head, block row); a 1-D grid
// with the batch index fastest, so dispatch follows the longest-first row
// order across the whole job. b/16 waves per key group, wave w owning query
// rows 16w..16w+15 of the block; NS key groups deal the row's blocks among
// themselves (k0 + sg, k0 + sg + NS, ...) and merge at the end. Each stored
// block is staged once into LDS for the waves of its group, K and V both
// row-major (contiguous 16-byte writes), and the next block is already in
// flight into registers while the current one is computed. Row strides were
// chosen by measuring the operand read patterns on gfx950; every operand
// read below is free of bank conflicts.
//
// Per 64-key sub-step and wave, with 16x16 MFMA tiles (fp32 16x16x4; bf16
// and fp16, the 16-bit types, 16x16x32):
//   S^T = K_c Q^T     A = K rows from LDS, B = the wave's Q rows (registers,
//                     loaded once). In the accumulator every lane then owns
//                     ONE query row (its column) and 4 keys per 16-key tile,
//                     so row max / sum are in-lane plus one butterfly over
//                     the 4 lane groups.
//   softmax           log2 domain (scale*log2(e) folded into Q for fp32, into
//                     one fma for 16-bit types); causal mask only on blocks that
//                     reach the diagonal; raw v_exp_f32. The reference max
//                     moves only when a block's max exceeds it by more than
//                     TAU (so p <= 2^TAU): numerator and denominator share it,
//                     so the result is exact, and most blocks skip the
//                     rescale of O.
//   O^T += V_c^T P^T  A = V^T, B = P^T straight from the score registers (no
//                     transpose); O^T also keeps one query row per lane, so
//                     the rescale is a per-lane scalar. fp32 takes one V
//                     element per lane and instruction (one 4-byte LDS read);
//                     16-bit types take 8 keys of one column per lane from two
//                     ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x
//                     16-column patch and every lane receives the 4 keys of
//                     its own column), so V never needs a transposed copy.
// The S^T register layout is also the layout of a row-major b x b block read
// with one 16-byte load per lane (row li, columns 16 jt + 4 g ..), which is
// how the SDD stores its scores and the DSD loads its P.
// 16-bit types: P is rounded to the operand type (RNE) for P.V and the row
// sum l adds up those rounded values (so the weights applied to V sum to one); O is rounded once
// at the end.
#ifndef BSA_ROWBLOCK_H
#define BSA_ROWBLOCK_H

#include <math.h>

#include <type_traits>

#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {  // each including translation unit instantiates its own modes

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;  // lazy-rescale headroom, log2 units

// MODE_DSDT is the DSD of the transposed block matrix (C = S^T-blocks x B):
// the same kernel walking block columns (CSC) and reading each stored block
// transposed.
// MODE_ATTN_MASKED is the fused attention with the dense additive masks (a
// separate instantiation, so that the unmasked kernel carries no mask code).
enum Mode { MODE_ATTN = 0, MODE_SDD = 1, MODE_DSD = 2, MODE_DSDT = 3, MODE_ATTN_MASKED = 4 };
constexpr bool is_attn(int mode) { return mode == MODE_ATTN || mode == MODE_ATTN_MASKED; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename E>
struct Cfg;
template <>
struct Cfg<float> {
  static constexpr int VEC = 4;   // elements per 16-byte vector
  static constexpr int KC = 16;   // contraction values per 16-byte lane vector group (4 groups x 4)
  typedef f32x4 Vec;
};
template <typename E>
struct Cfg16 {
  static constexpr int VEC = 8;
  static constexpr int KC = 32;
  typedef typename H16<E>::V8 Vec;
};
template <>
struct Cfg<bf16_t> : Cfg16<bf16_t> {};
template <>
struct Cfg<f16_t> : Cfg16<f16_t> {};

// padded LDS row strides (elements), measured free of bank conflicts for the
// operand reads of the kernel: K rows 32 mod 256 bytes; V rows 16 mod 64
// bytes (fp32, one 4-byte read per lane) or 32 mod 256 bytes (16-bit types,
// transposing 8-byte reads)
template <typename E, int BLK, int D, int MODE>
struct Lds {
  using St = typename Elem<E>::storage;
  static constexpr int KSTR = D + 32 / (int)sizeof(St);
  static constexpr int VSTR = std::is_same<E, float>::value ? D + 4 : D + 16;
  static constexpr int KBUF = (MODE == MODE_DSD || MODE == MODE_DSDT) ? 0 : BLK * KSTR;  // per key group
  static constexpr int VBUF = MODE == MODE_SDD ? 0 : BLK * VSTR;
  static constexpr size_t STAGE = (size_t)(KBUF + VBUF) * sizeof(St);  // bytes per key group
};

// Q, K, V, O: [Z][H][N][D] dense operands; S: [Z][nnz][BLK][BLK] fp32 block
// values (SDD output, DSD input). MODE_ATTN uses Q, K, V -> O; MODE_SDD
// uses Q (= A), K (= B) -> S; MODE_DSD uses S (= P), V (= B) -> O (= C);
// MODE_DSDT takes the column tables (col_ptr, row_idx, col_order and blk_id
// in place of row_ptr, col_idx, row_order and the identity) with nbr and nbc
// swapped, and reads each block of S transposed.
template <typename E, int BLK, int D, bool CAUSAL, int NS, int MODE>
__global__ __launch_bounds__(BLK * 4 * NS) void k_rowblock(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, const int32_t* __restrict__ row_order,
    const typename Elem<E>::storage* __restrict__ Q, const typename Elem<E>::storage* __restrict__ K,
    const typename Elem<E>::storage* __restrict__ V, typename Elem<E>::storage* __restrict__ O,
    float* __restrict__ S, const int32_t* __restrict__ blk_id, const int32_t* __restrict__ band, int band_n, int Z,
    int H, int nbr, int nbc, int64_t nnz, float c, const float* __restrict__ amask,
    const float* __restrict__ kpmask, float* __restrict__ lse, const int32_t* __restrict__ row_order_h,
    int grouped) {
  using St = typename Elem<E>::storage;
  using Vec = typename Cfg<E>::Vec;
  constexpr bool BF = !std::is_same<E, float>::value;  // a 16-bit element type (bf16, fp16)
  constexpr bool ATTN = is_attn(MODE);
  constexpr bool MASKED = MODE == MODE_ATTN_MASKED;
  constexpr bool DSDT = MODE == MODE_DSDT;
  constexpr bool HASK = MODE != MODE_DSD && !DSDT;  // score product (Q, K staged)
  constexpr bool HASV = MODE != MODE_SDD;  // P.V product (V staged)
  constexpr int VEC = Cfg<E>::VEC, KC = Cfg<E>::KC;
  constexpr int NW = BLK / 16, NT = 64 * NW;  // waves / threads of one key group
  constexpr int NQ = D / KC;                  // Q fragments per lane
  // Staging of the next block: split (K during the score product, V during
  // softmax and P.V, one matrix in registers at a time) where registers are
  // the limit, else both at the start of a step, hidden by the whole step.
  constexpr bool SPLIT = ATTN && BF && D == 128;
  constexpr int KS = BLK < 64 ? BLK : 64;  // keys per sub-step
  constexpr int NSUB = BLK / KS;
  constexpr int NJT = KS / 16;             // 16-key tiles per sub-step
  constexpr int NNT = D / 16;              // 16-column tiles of O
  // DSD with two sub-steps per block: P of the next sub-step is loaded one
  // sub-step ahead into the other of two register sets
  constexpr bool PFP = MODE == MODE_DSD && NSUB == 2 && BF;
  constexpr int KSTR = Lds<E, BLK, D, MODE>::KSTR;
  constexpr int VSTR = Lds<E, BLK, D, MODE>::VSTR;
  constexpr int KBUF = Lds<E, BLK, D, MODE>::KBUF, VBUF = Lds<E, BLK, D, MODE>::VBUF;
  constexpr int CPR = D / VEC;         // 16-byte chunks per row
  constexpr int KCH = BLK * CPR / NT;  // chunks per thread and matrix (D / (4 VEC))
  static_assert(KCH >= 1 && BLK * CPR % NT == 0, "staging");
  constexpr int SLOT = 64 * ((ATTN ? 2 : 0) + 4 * NNT);  // floats per wave for the final merge
  // one LDS array: the K stages of the NS groups, then their V stages; the
  // final merge of the groups reuses it from the start
  constexpr int MERGE_ELEMS = (MODE == MODE_SDD || NS == 1) ? 0 : (NS - 1) * NW * SLOT * 4 / (int)sizeof(St);
  constexpr int LDS_ELEMS = NS * (KBUF + VBUF) > MERGE_ELEMS ? NS * (KBUF + VBUF) : MERGE_ELEMS;
  static_assert((KBUF * sizeof(St)) % 16 == 0, "16-byte aligned V stages");

  __shared__ __attribute__((aligned(16))) St lds[LDS_ELEMS];
  St* const Ks = lds;
  St* const Vs = lds + NS * KBUF;

  const int tid_all = threadIdx.x;
  const int sg = __builtin_amdgcn_readfirstlane(tid_all / NT);  // key group of this wave
  const int tid = tid_all % NT;                                 // thread index inside the key group
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);    // query tile; uniform keeps mask tests scalar
  const int lane = tid & 63;
  St* const Kg = Ks + sg * KBUF;
  St* const Vg = Vs + sg * VBUF;
  const int li = lane & 15, g = lane >> 4;
  // Which block row: with `grouped`, XCD-aware and grouped by (batch, head),
  // the head's rows longest first (the head's K or V blocks, which its rows
  // read again and again, stay in the XCD's L2 while its rows are in
  // flight); otherwise longest first across the whole job, batch index
  // fastest (the long rows start first).
  int hr, z;
  if (grouped) {
    const int unit = xcd_unit(blockIdx.x, gridDim.x);
    const int zhu = unit / nbr;
    z = zhu / H;
    hr = row_order_h[(zhu % H) * nbr + unit % nbr];
  } else {
    hr = row_order[blockIdx.x / Z];
    z = blockIdx.x % Z;
  }
  const int h = hr / nbr, r = hr % nbr;
  // The row's blocks: positions k0..k1-1 of the column table, or, for a
  // slope-1 ACSR layout (band != null, attention only), columns r + band[i]
  // for the offsets that keep the column on the grid (found by two binary
  // searches in the sorted offsets; same ascending order as the table)
  int k0, k1, boff = 0;
  if (band != nullptr) {
    auto first_at_least = [&](int v) {
      int lo = 0, hi = band_n;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (band[mid] < v) lo = mid + 1;
        else hi = mid;
      }
      return lo;
    };
    boff = first_at_least(-(hr % nbr));
    k0 = 0;
    // causal attention: no column after the row either (offsets up to 0)
    const int end = nbc - (hr % nbr);
    k1 = first_at_least((ATTN && CAUSAL && end > 1) ? 1 : end) - boff;
  } else {
    k0 = row_ptr[hr];
    k1 = row_ptr[hr + 1];
    // causal attention: key blocks after the row (wholly above the
    // diagonal) are neither staged nor computed
    if constexpr (ATTN && CAUSAL) trim_causal<false>(col_idx, hr % nbr, k0, k1);
  }
  auto col_of = [&](int kk) { return band != nullptr ? hr % nbr + band[boff + kk] : col_idx[kk]; };
  const int64_t zh = (int64_t)z * H + h;
  const int64_t Nq = (int64_t)nbr * BLK, Nk = (int64_t)nbc * BLK;
  const int q_lo = r * BLK + wave * 16;  // first query row of this wave
  const int q_index = q_lo + li;         // this lane's query row
  const St* Kz = K + zh * Nk * D;
  const St* Vz = V + zh * Nk * D;
  // this lane's row of a stored block in S: row wave*16 + li, columns 4g..
  const int64_t s_lane = (int64_t)(wave * 16 + li) * BLK + 4 * g;

  // ---- Q as B fragments; attention folds scale*log2(e) in (fp32) or only
  // its sign (16-bit types, exact); the SDD uses Q as is
  Vec qf[HASK ? NQ : 1];
  float cs = 1.f;
  if constexpr (HASK) {
    const St* pq = Q + (zh * Nq + q_index) * D + g * VEC;
#pragma unroll
    for (int u = 0; u < NQ; ++u) qf[u] = *reinterpret_cast<const Vec*>(pq + u * KC);
    if constexpr (ATTN && BF) {
      const float sgn = c > 0.f ? 1.f : (c < 0.f ? -1.f : 0.f);
      if (sgn != 1.f) {
#pragma unroll
        for (int u = 0; u < NQ; ++u)
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[u][e] = H16<E>::cvt((float)qf[u][e] * sgn);
      }
      cs = (c == 0.f) ? 1.f : fabsf(c);
    } else if constexpr (ATTN) {
#pragma unroll
      for (int u = 0; u < NQ; ++u) qf[u] *= c;
    }
  }

  // dense additive masks (attention): the scores get s * cs + log2(e) *
  // mask and are in log2 units from then on
  const float cs_in = cs;
  if constexpr (MASKED) cs = 1.f;

  // ---- staging of one block: K and V use the same chunk mapping; with
  // SPLIT they share registers (held at different times)
  Vec stg[KCH];
  Vec stv[(HASK && HASV && !SPLIT) ? KCH : 1];
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
  auto stage_load_to = [&](Vec* rg, const St* base, int cb) {
    const St* src = base + (int64_t)cb * BLK * D;  // uniform
#pragma unroll
    for (int i = 0; i < KCH; ++i) rg[i] = *reinterpret_cast<const Vec*>(src + goff[i]);
  };
  auto stage_store_from = [&](const Vec* rg, St* dst, const int* off) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) *reinterpret_cast<Vec*>(&dst[off[i]]) = rg[i];
  };
  // the next block's matrices in registers, without SPLIT: K in stg and V
  // in stv (attention), or the one matrix in stg (SDD: K, DSD: V)
  auto load_next = [&](int cb) {
    if constexpr (HASK) stage_load_to(stg, Kz, cb);
    if constexpr (HASV) stage_load_to(HASK ? stv : stg, Vz, cb);
  };
  auto store_next = [&]() {
    if constexpr (HASK) stage_store_from(stg, Kg, koff);
    if constexpr (HASV) stage_store_from(HASK ? stv : stg, Vg, voff);
  };

  // PFP: P of sub-step x of stored block kk in the score-register layout
  // (this lane: query wave*16 + li, keys 64x + 16 jt + 4 g + rr)
  f32x4 pset[PFP ? 2 : 1][PFP ? NJT : 1];
  auto load_p = [&](int kk, int x, f32x4 (&dst)[PFP ? NJT : 1]) {
    if constexpr (PFP) {
      const float* src = S + ((int64_t)z * nnz + kk) * (BLK * BLK) + s_lane + x * KS;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) dst[jt] = *reinterpret_cast<const f32x4*>(src + 16 * jt);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[HASV ? NNT : 1];
#pragma unroll
  for (int nt = 0; nt < (HASV ? NNT : 1); ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Without SPLIT a step is: barrier, store the staged block, barrier, load
  // the next block (in flight during the compute), compute. With SPLIT: K of
  // the next block is loaded during the score product and stored once every
  // wave is past it; V of the next block is loaded then and stored once
  // every wave is past P.V.
  const int nsteps = (k1 - k0 + NS - 1) / NS;
  if (k0 + sg < k1) {
    if constexpr (SPLIT) {
      stage_load_to(stg, Kz, col_of(k0 + sg));
      stage_store_from(stg, Kg, koff);
      stage_load_to(stg, Vz, col_of(k0 + sg));
      stage_store_from(stg, Vg, voff);
    } else {
      load_next(col_of(k0 + sg));
    }
  }
  if constexpr (SPLIT) __syncthreads();
  if constexpr (PFP) {
    if (k0 + sg < k1) load_p(k0 + sg, 0, pset[0]);
    // the loads so far have arrived before the loop, so that the compiler's
    // waits inside it count only the loads of the loop
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
  }
  for (int step = 0; step < nsteps; ++step) {
    const int kk = k0 + step * NS + sg;
    const bool valid = kk < k1;
    const bool has_next = kk + NS < k1;
    const int cb_next = has_next ? col_of(kk + NS) : 0;
    if constexpr (!SPLIT) {
      __syncthreads();  // every wave is done with the previous blocks in LDS
      if (valid) store_next();
      __syncthreads();
      if constexpr (PFP) {
        // issued on every step, a block of this row standing in when there is
        // no next one (never stored: the next step is not valid), so that
        // the compiler counts the same loads on every path
        load_next(has_next ? cb_next : col_of(valid ? kk : k0));
      } else if (has_next) {
        load_next(cb_next);
      }
    } else {
      if (has_next) stage_load_to(stg, Kz, cb_next);
    }
    const int cb = valid ? col_of(kk) : 0;
    // blocks whose every key is after every query of this wave add nothing
    const bool compute = valid && !(ATTN && CAUSAL && cb * BLK > q_lo + 15);
    const bool mask_block = ATTN && CAUSAL && (cb * BLK + BLK - 1 > q_lo);
    const int64_t blk = DSDT ? (valid ? (int64_t)blk_id[kk] : 0) : (int64_t)kk;  // stored block id
    float* const s_blk = S + ((int64_t)z * nnz + blk) * (BLK * BLK) + s_lane;
    // DSDT: element (i, j) of the transposed block is S[j][i]; this lane
    // needs keys kofs + 16 jt + 4 g + rr of query wave*16 + li
    const float* const st_blk = S + ((int64_t)z * nnz + blk) * (BLK * BLK) + (int64_t)(4 * g) * BLK + wave * 16 + li;

#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const int kofs = sub * KS;  // first key of this sub-step within the block
      // s[jt][rr] = score of (query li, key kofs + 16 jt + 4 g + rr)
      f32x4 s[NJT];

      // ---- S^T = K Q^T (attention, SDD); the K operands of tile jt+1 are
      // read from LDS while tile jt is multiplied (fp32)
      if constexpr (HASK) {
        const St* kbase = &Kg[(kofs + li) * KSTR + g * VEC];
        if (!compute) {
        } else if constexpr (BF) {
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) {
            s[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < NQ; ++u) {
              const Vec a = *reinterpret_cast<const Vec*>(kbase + 16 * jt * KSTR + u * KC);
              s[jt] = H16<E>::mfma16(a, qf[u], s[jt]);
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
      }

      if constexpr (MODE == MODE_SDD) {
        // the raw scores are the output
        if (compute) {
          if constexpr (BLK <= 64) {
            // written once: streaming stores, 16 rows x 64 bytes per
            // instruction (the lane exchange below measured 4-11% slower
            // here)
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt)
              __builtin_nontemporal_store(s[jt], reinterpret_cast<f32x4*>(s_blk + kofs + 16 * jt));
          } else {
            // 128-blocks: tiles 2jp and 2jp + 1 as two streaming stores of 8
            // rows x 32 keys, whole 128-byte lines: lanes li and li ^ 8 swap
            // one tile (lane li < 8 keeps row li's first 16 keys and takes row
            // li + 8's; lane li >= 8 keeps row li's last 16 and takes row
            // li - 8's). Measured on random_b128_bf16: 1.73 ms, against 1.84
            // with plain stores of the same lines and 2.08 with plain stores
            // of 16 rows x 64 bytes (streaming stores of those: 2.9).
            const bool lo = li < 8;
            float* const s_w = s_blk - (int64_t)li * BLK;  // row wave*16 of the block, column 4g
            const int row = li & 7;
#pragma unroll
            for (int jp = 0; jp < NJT / 2; ++jp) {
              const f32x4 a = s[2 * jp], b = s[2 * jp + 1];
              const f32x4 x = lo ? b : a;
              const f32x4 y = {__shfl_xor(x[0], 8), __shfl_xor(x[1], 8), __shfl_xor(x[2], 8), __shfl_xor(x[3], 8)};
              const int col = kofs + 32 * jp + (lo ? 0 : 16);
              __builtin_nontemporal_store(lo ? a : y, reinterpret_cast<f32x4*>(s_w + (int64_t)row * BLK + col));
              __builtin_nontemporal_store(lo ? y : b, reinterpret_cast<f32x4*>(s_w + (int64_t)(row + 8) * BLK + col));
            }
          }
        }
        continue;
      }
      if constexpr (DSDT) {
        if (compute) {
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) s[jt][rr] = st_blk[(int64_t)(kofs + 16 * jt + rr) * BLK];
        }
      }
      if constexpr (PFP) {
        // P of the other sub-step into the other set (this block's second
        // half, then the next block's first half, a block of this row
        // standing in past the end), then this sub-step's P, loaded one
        // sub-step ago
        if (sub == 0) load_p(valid ? kk : k0, 1, pset[1]);
        else load_p(has_next ? kk + NS : k0, 0, pset[0]);
        if (compute) {
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) s[jt] = pset[sub][jt];
        }
      } else if constexpr (MODE == MODE_DSD) {
        // P block rows straight into the score-register layout
        if (compute) {
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) s[jt] = *reinterpret_cast<const f32x4*>(s_blk + kofs + 16 * jt);
        }
      }

      if (SPLIT && sub == NSUB - 1) {
        __syncthreads();  // every wave is past the score product: K of the next block may land
        if (has_next) {
          stage_store_from(stg, Kg, koff);
          stage_load_to(stg, Vz, cb_next);
        }
      }
      if (!compute) continue;

      if constexpr (ATTN) {
        // ---- dense additive masks: s * cs + log2(e) * mask, after which the
        // scores are in log2 units (cs becomes 1)
        if constexpr (MASKED) {
          const int64_t key0 = (int64_t)cb * BLK + kofs + 4 * g;
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) {
            f32x4 mv = {0.f, 0.f, 0.f, 0.f};
            if (amask != nullptr) mv = *reinterpret_cast<const f32x4*>(amask + q_index * Nk + key0 + 16 * jt);
            if (kpmask != nullptr) mv += *reinterpret_cast<const f32x4*>(kpmask + z * Nk + key0 + 16 * jt);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) s[jt][rr] = fmaf(mv[rr], kLog2e, s[jt][rr] * cs_in);
          }
        }
        // ---- causal mask, block max (raw scores; cs > 0), lazy rescale, exp2
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
        mx = rows4_max(mx);
        const float m_blk = mx * cs;
        const bool upd = m_blk > m_run + kTau;
        if (__builtin_amdgcn_ballot_w64(upd) != 0) {  // wave-uniform
          const float m_new = upd ? m_blk : m_run;
          // lanes that keep their max keep their sums (a row that has seen
          // nothing yet, m_run = -inf, would otherwise get exp2(-inf + inf));
          // an update has a finite m_new, so alpha is 0 when m_run = -inf
          const float alpha = upd ? fast_exp2(m_run - m_new) : 1.f;
          l_run *= alpha;
#pragma unroll
          for (int nt = 0; nt < NNT; ++nt) o[nt] *= alpha;
          m_run = m_new;
        }
        const float m_sub = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) s[jt][rr] = fast_exp2(fmaf(s[jt][rr], cs, -m_sub));
        if constexpr (!BF) {
          // 16-bit types sum the rounded P below, two values per instruction
          float ls = 0.f;
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) ls += s[jt][rr];
          l_run += ls;
        }
      }

      // ---- O^T[n][query] += V^T[n][keys] P^T[keys][query]
      if constexpr (BF) {
        // lane (g, j = 4k + m) points at row 16h + 4g + k, columns 4m.. of
        // the n-tile; it gets back keys 16h + 4g + 0..3 of column nt*16 + li
        const u16* vb = &Vg[(kofs + 4 * g + (li >> 2)) * VSTR + 4 * (li & 3)];
        // attention: the row sum l adds up P as rounded for the product (the
        // weights that multiply V), two per v_dot2 against (1, 1)
        using HT = H16<E>;
        using V8 = typename HT::V8;
        using V4 = typename HT::V4;
        float ls = 0.f;
        const typename HT::V2 ones = {HT::cvt(1.f), HT::cvt(1.f)};
        auto sum_p = [&](const V8& pb) {
          if constexpr (ATTN) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) ls = HT::dot2(typename HT::V2{pb[e], pb[e + 1]}, ones, ls);
          }
        };
        if constexpr (NJT >= 2) {
          // operands read right before use: the 16-bit kernel is register
          // bound (two 8-wave workgroups per CU need <= 128 VGPRs)
#pragma unroll
          for (int jp = 0; jp < NJT / 2; ++jp) {
            const V8 pb = {HT::cvt(s[2 * jp][0]),     HT::cvt(s[2 * jp][1]),     HT::cvt(s[2 * jp][2]),
                           HT::cvt(s[2 * jp][3]),     HT::cvt(s[2 * jp + 1][0]), HT::cvt(s[2 * jp + 1][1]),
                           HT::cvt(s[2 * jp + 1][2]), HT::cvt(s[2 * jp + 1][3])};
            sum_p(pb);
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) {
              const V4 a0 = lds_read_tr16_as<V4>(vb + (32 * jp) * VSTR + nt * 16);
              const V4 a1 = lds_read_tr16_as<V4>(vb + (32 * jp + 16) * VSTR + nt * 16);
              const V8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
              o[nt] = HT::mfma16(a, pb, o[nt]);
            }
          }
        } else {  // a single 16-key tile: the other half of the k range is zero
          const typename HT::T zb = HT::cvt(0.f);
          const V8 pb = {HT::cvt(s[0][0]), HT::cvt(s[0][1]), HT::cvt(s[0][2]), HT::cvt(s[0][3]), zb, zb, zb, zb};
          sum_p(pb);
#pragma unroll
          for (int nt = 0; nt < NNT; ++nt) {
            const V4 a0 = lds_read_tr16_as<V4>(vb + nt * 16);
            const V8 a = {a0[0], a0[1], a0[2], a0[3], zb, zb, zb, zb};
            o[nt] = HT::mfma16(a, pb, o[nt]);
          }
        }
        if constexpr (ATTN) l_run += ls;
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
              for (int nt = 0; nt < NNT; ++nt)
                va[(jt + 1) & 1][rr][nt] = vbase[(16 * (jt + 1) + rr) * VSTR + nt * 16];
          }
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt)
              o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[jt & 1][rr][nt], s[jt][rr], o[nt], 0, 0, 0);
        }
      }
    }  // sub-step
    if constexpr (SPLIT) {
      __syncthreads();  // every wave is past P.V: V of the next block may land
      if (has_next) stage_store_from(stg, Vg, voff);
      // with sub-steps, the first P.V of the next block precedes its
      // mid-block barrier, so V must be visible before the next step starts
      if constexpr (NSUB > 1) __syncthreads();
    }
  }
  if constexpr (MODE == MODE_SDD) return;

  // ---- merge the key groups through LDS into group 0: attention rescales
  // each side's (l, O) by exp2(m_side - m_max); the DSD adds the partial sums
  if constexpr (NS > 1) {
    float* red = reinterpret_cast<float*>(lds);
    __syncthreads();
    if (sg > 0) {
      float* slot = red + ((sg - 1) * NW + wave) * SLOT;
      if constexpr (ATTN) {
        slot[lane] = m_run;
        slot[64 + lane] = l_run;
      }
#pragma unroll
      for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) slot[(ATTN ? 128 : 0) + (nt * 4 + e) * 64 + lane] = o[nt][e];
    }
    __syncthreads();
    if (sg > 0) return;
#pragma unroll
    for (int s2 = 1; s2 < NS; ++s2) {
      const float* slot = red + ((s2 - 1) * NW + wave) * SLOT;
      if constexpr (ATTN) {
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
      } else {
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[nt][e] += slot[(nt * 4 + e) * 64 + lane];
      }
    }
  }

  // ---- finish: attention divides by l (summed over the 4 lane groups);
  // O^T rows are written 4 columns per store
  float inv = 1.f;
  if constexpr (ATTN) {
    l_run = rows4_sum(l_run);
    inv = (l_run > 0.f) ? 1.0f / l_run : 0.f;
    // the row's log-sum-exp in natural-log units: l is a sum of
    // exp2(x - m_run) with x and m_run in log2 units, l >= 1 when the row
    // saw anything (its largest term is at least 1)
    if (lse != nullptr && g == 0)
      lse[zh * Nq + q_index] = (l_run > 0.f) ? (m_run + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
  }
  St* po = O + (zh * Nq + q_index) * D + 4 * g;
#pragma unroll
  for (int nt = 0; nt < NNT; ++nt) {
    if constexpr (BF) {
      using HT = H16<E>;
      *reinterpret_cast<typename HT::V4*>(po + nt * 16) = typename HT::V4{
          HT::cvt(o[nt][0] * inv), HT::cvt(o[nt][1] * inv), HT::cvt(o[nt][2] * inv), HT::cvt(o[nt][3] * inv)};
    } else {
      *reinterpret_cast<f32x4*>(po + nt * 16) = o[nt] * inv;
    }
  }
}

struct Args {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* S;
  int Z;
  float c;
  bool causal;
  bool use_band = false;  // attention on a slope-1 ACSR layout: computed columns
  const float* am = nullptr;  // dense additive masks (attention)
  const float* kp = nullptr;
  float* lse = nullptr;  // optional row log-sum-exp output (attention)
};

template <typename E, int BLK, int D, int NS, int MODE>
int launch_ns(const bs_layout* L, const Args& a, hipStream_t s) {
  using St = typename Elem<E>::storage;
  constexpr bool T = MODE == MODE_DSDT;  // column-wise
  const int units = T ? L->nbc : L->nbr;
  const dim3 grid(L->H * units * a.Z), block(BLK * 4 * NS);
  const int32_t* ptr = T ? L->col_ptr : L->row_ptr;
  const int32_t* idx = T ? L->row_idx : L->col_idx;
  const int32_t* order = T ? L->col_order : L->row_order;
  const int32_t* order_h = T ? L->col_order_h : L->row_order_h;
  // head-grouped XCD order for the SDD and DSD modes with 16-bit operands
  // and rows (columns) of similar length: the longest, split over the NS
  // groups, is at most a quarter of a workgroup slot's share (two slots per
  // CU). Measured on random_b128_bf16: SDD +16%, DSD +5%; the fp32 workloads
  // ran up to 55% slower with it (their longest-first order already reuses
  // K or V across heads), so they keep longest first.
  const double per_slot = (double)a.Z * (double)L->nnz / (2.0 * L->num_cus);
  const int max_len = T ? L->max_col_len : L->max_row_len;
  const int grouped = (!is_attn(MODE) && !std::is_same<E, float>::value && 4.0 * max_len / NS <= per_slot) ? 1 : 0;
  const int32_t* bid = T ? L->blk_id : nullptr;
  const int nb_out = T ? L->nbc : L->nbr, nb_in = T ? L->nbr : L->nbc;
  // the fused kernel computes slope-1 ACSR columns (the other modes index S by
  // the table position, so they keep the table)
  const int32_t* band = (is_attn(MODE) && a.use_band) ? L->band_off : nullptr;
  const int band_n = band ? L->band_n : 0;
  if (is_attn(MODE) && a.causal)
    hipLaunchKernelGGL((k_rowblock<E, BLK, D, true, NS, MODE>), grid, block, 0, s, ptr, idx, order, (const St*)a.Q,
                       (const St*)a.K, (const St*)a.V, (St*)a.O, a.S, bid, band, band_n, a.Z, L->H, nb_out, nb_in,
                       L->nnz, a.c, a.am, a.kp, a.lse, order_h, grouped);
  else
    hipLaunchKernelGGL((k_rowblock<E, BLK, D, false, NS, MODE>), grid, block, 0, s, ptr, idx, order,
                       (const St*)a.Q, (const St*)a.K, (const St*)a.V, (St*)a.O, a.S, bid, band, band_n, a.Z, L->H,
                       nb_out, nb_in, L->nnz, a.c, a.am, a.kp, a.lse, order_h, grouped);
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

// Key groups per workgroup. With one group, several workgroups share a CU,
// so a row of n blocks needs ~share*n block-times of its CU while the CU's
// whole share of the job is Z*nnz/CUs block-times: once the longest row
// exceeds that, it sets the end of the kernel. NS groups cut the row's own
// time by NS (the groups run its blocks side by side and merge at the end).
// The share was set by measurement: 2 for the fused attention (causal_b64
// NS = 1 and bigbird_b64 NS = 2 came out 4% and 13% faster than with 4),
// 4 for the SDD and DSD modes (2 made the DSD up to 18% slower).
inline int pick_key_groups(const bs_layout* L, int Z, int max_ns, int max_len, double share) {
  const double per_cu = (double)Z * (double)L->nnz / L->num_cus;
  int ns = 1;
  while (ns < max_ns && share * max_len / ns > per_cu) ns *= 2;
  return ns;
}

template <typename E, int BLK, int D, int MODE>
int run(const bs_layout* L, const Args& a, hipStream_t s) {
  // largest key-group count (up to 4, and 1024 threads) whose LDS fits in 160 KiB
  constexpr size_t stage = Lds<E, BLK, D, MODE>::STAGE;
  // four groups of a 64-block row are 1024 threads, at most 128 VGPRs a
  // lane: the 16-bit d = 128 attention and the masked attention need more
  // (they spilled), so they stop at two
  constexpr bool fits4 = !(MODE == MODE_ATTN && !std::is_same<E, float>::value && D == 128) && MODE != MODE_ATTN_MASKED;
  constexpr int max_ns = (BLK <= 64 && 4 * stage <= 160 * 1024 && fits4)
                             ? 4
                             : ((BLK <= 64 && 2 * stage <= 160 * 1024) ? 2 : 1);
  const int ns = pick_key_groups(L, a.Z, max_ns, MODE == MODE_DSDT ? L->max_col_len : L->max_row_len,
                                 is_attn(MODE) ? 2.0 : 4.0);
  if constexpr (max_ns >= 4) {
    if (ns >= 4) return launch_ns<E, BLK, D, 4, MODE>(L, a, s);
  }
  if constexpr (max_ns >= 2) {
    if (ns >= 2) return launch_ns<E, BLK, D, 2, MODE>(L, a, s);
  }
  return launch_ns<E, BLK, D, 1, MODE>(L, a, s);
}

template <typename E, int D, int MODE>
int run_b(const bs_layout* L, const Args& a, hipStream_t s) {
  switch (L->block) {
    case 16: return run<E, 16, D, MODE>(L, a, s);
    case 32: return run<E, 32, D, MODE>(L, a, s);
    case 64: return run<E, 64, D, MODE>(L, a, s);
    case 128: return run<E, 128, D, MODE>(L, a, s);
  }
  return fail(BS_ERR_UNSUPPORTED, "block must be 16, 32, 64 or 128");
}

template <int MODE>
int run_mode(const bs_layout* L, const Args& a, int d, bs_dtype dt, hipStream_t s) {
  if (dt == BS_BF16) return d == 64 ? run_b<bf16_t, 64, MODE>(L, a, s) : run_b<bf16_t, 128, MODE>(L, a, s);
  if (dt == BS_F16) return d == 64 ? run_b<f16_t, 64, MODE>(L, a, s) : run_b<f16_t, 128, MODE>(L, a, s);
  return d == 64 ? run_b<float, 64, MODE>(L, a, s) : run_b<float, 128, MODE>(L, a, s);
}

}  // namespace
}  // namespace bsa

#endif  // BSA_ROWBLOCK_H
