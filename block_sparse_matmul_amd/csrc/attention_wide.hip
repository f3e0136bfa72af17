// Fused block-sparse attention, 16-bit operands (bf16 or fp16), blocks of
// 32 to 128: the same computation as the row-block kernel (SDD ->
// block-sparse softmax -> DSD of Triton issue 117, "question on
// blocksparse", with the streaming softmax of the Triton tutorial, Puzzles 8
// and 9), laid out for the 16-bit matrix cores.
//
// What differs from the row-block kernel:
//  * each wave owns 32 query rows (two 16-row tiles), so every K or V
//    operand read from LDS feeds two MFMAs: half the LDS read traffic per
//    flop, which is what bounds the 16-row layout with 16-bit operands;
//  * blocks are staged with LDS DMA (buffer_load_dwordx4 ... lds: every
//    lane moves 16 bytes from its own offset in the (batch, head)'s K or V
//    into consecutive LDS slots), so staging needs no registers and no LDS
//    store instructions. The buffer form takes a scalar base and offset and
//    a 32-bit per-lane offset; the global form needed a 64-bit address add
//    per lane and transfer (1.5-2% slower on random_b128_bf16).
//    Rows are stored unpadded with their 16-byte chunks XOR-swizzled by row
//    (d = 128: slot = chunk ^ ((2 row) & 14); d = 64: slot = chunk ^
//    (((row >> 1) ^ row) & 7)), which keeps the K reads (16 bytes per lane)
//    and the transposing V reads (ds_read_b64_tr_b16) free of bank
//    conflicts, as measured on gfx950;
//  * K and V are staged by sub-steps of 64 keys. With one sub-step per
//    block, V of the block is fetched at the top of the step (hidden by the
//    score product) and K of the next block once every wave is past its
//    score product; with two (128-blocks), the K and V of the next sub-step
//    are fetched together during the current one, into the slots of the
//    previous one, one barrier per sub-step.
//
// Per 64-key sub-step and wave (16x16x32 bf16 / fp16 MFMA tiles, as in the
// row-block kernel): S^T = K Q^T for both query tiles from one K read;
// softmax in the log2 domain with lazy rescale; O^T += V^T P^T for both
// tiles from one pair of transposing V reads. The row sum adds up P as
// rounded to the operand type for the product (v_dot2 against (1, 1)).
#include <math.h>

#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

constexpr float kLog2eB = 1.4426950408889634f;
constexpr float kLn2B = 0.6931471805599453f;
constexpr float kTauB = 8.0f;  // lazy-rescale headroom, log2 units
// fourth word of a raw buffer resource on gfx9 (32-bit data format, no
// swizzle, no index stride)
constexpr int kRsrcWord3 = 0x00020000;

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// fp8 operands: tag of the element type in which Q and K are OCP FP8 E4M3
// (one byte each) and the score product runs on the fp8 matrix cores
// (v_mfma_f32_16x16x128_f8f6f4, exact products, fp32 accumulation), while V,
// P and O stay bf16
struct f8_t {};
template <typename E>
struct WideTypes {
  typedef E PV;  // element type of V, P and O
  static constexpr bool F8 = false;
};
template <>
struct WideTypes<f8_t> {
  typedef bf16_t PV;
  static constexpr bool F8 = true;
};

template <int D>
struct Swz;
template <>
struct Swz<128> {  // 256-byte rows, 16 chunks
  static __device__ __forceinline__ int f(int r) { return (2 * r) & 14; }
};
template <>
struct Swz<64> {  // 128-byte rows, 8 chunks
  static __device__ __forceinline__ int f(int r) { return ((r >> 1) ^ r) & 7; }
};

template <int BLK, int D, int RBK = 2 * D>
struct WideCfg {
  static constexpr int NW = BLK / 32;            // waves per key group
  static constexpr int RB = D * 2;               // bytes per V row
  static constexpr int SB = BLK * RB;            // bytes per staged V block
  static constexpr int SBK = BLK * RBK;          // bytes per staged K block (RBK bytes per K row)
  static constexpr int NNT = D / 16;             // 16-column tiles of O
  static constexpr int SLOT = 64 * (2 + 4 * NNT);  // floats per wave and tile for the merge
  // LDS of a workgroup with ns key groups: K stages and V stages; the merge
  // (one query tile at a time) reuses the K stages
  static constexpr size_t bytes(int ns) { return (size_t)ns * (SB + SBK); }
  static constexpr bool merge_fits(int ns) { return ns == 1 || (size_t)(ns - 1) * NW * SLOT * 4 <= (size_t)ns * SBK; }
};

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt and lgkmcnt left at "no wait")
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_vmcnt0() { wait_vmcnt<0>(); }
// workgroup barrier after this wave's LDS operations, without the memory
// fence of __syncthreads (which also waits for every LDS DMA transfer in
// flight): the transfers are paced by the explicit vmcnt waits
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// MASKED: the dense additive masks (amask [nbr*b][nbc*b], kpmask [Z][nbc*b],
// either may be null) are read at the start of each sub-step, one 16-byte
// vector per lane, 16-key tile and query tile, while the score product
// runs. The transfers above are paced by counting the vector-memory
// operations in flight; the mask reads join that count, which can only
// make a wait wait for more (every operation completes in order), never
// for less.
//
// BAND: K/V shared across block rows on a slope-1 ACSR layout (the sharing
// plan of the layout; see attention_band.hip for the plan): the NS = 2
// groups of the workgroup take block rows r0 and r0 + stride instead of
// dealing one row's blocks; they walk the union of the two rows' columns
// (r0 + uoff[i]) together, through one K and V stage that group 0 fills,
// and the waves of a row compute on the blocks whose mask bit is theirs.
// Each row adds up its own blocks in ascending order with the same
// per-block code, so no merge is needed.
template <typename E, int BLK, int D, bool CAUSAL, int NS, bool MASKED, bool BAND = false>
__global__ __launch_bounds__(BLK * 2 * NS) void k_attn_wide(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, const int32_t* __restrict__ row_order,
    const int32_t* __restrict__ row_order_h, const void* __restrict__ Qv, const void* __restrict__ Kv,
    const u16* __restrict__ V, u16* __restrict__ O, int Z, int H, int nbr, int nbc, float c, int grouped,
    float* __restrict__ lse, const float* __restrict__ amask, const float* __restrict__ kpmask,
    const int32_t* __restrict__ uoff = nullptr, const int32_t* __restrict__ umask = nullptr,
    const int32_t* __restrict__ grp = nullptr, int nu = 0, int stride = 0) {
  static_assert(!BAND || (NS == 2 && !MASKED), "K/V sharing: two rows a workgroup, no dense masks");
  constexpr bool F8 = WideTypes<E>::F8;
  constexpr int RBK = F8 ? D : 2 * D;  // bytes per K row
  using Cfg = WideCfg<BLK, D, RBK>;
  using HT = H16<typename WideTypes<E>::PV>;
  using V8 = typename HT::V8;
  using V4 = typename HT::V4;
  using V2 = typename HT::V2;
  constexpr int NW = Cfg::NW, NT = 64 * NW;
  constexpr int NQ = D / 32;         // Q fragments per lane and tile
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int RB = Cfg::RB;
  constexpr int RPI = 1024 / RB;     // V rows per DMA instruction (64 lanes x 16 bytes)
  constexpr int RPIK = 1024 / RBK;   // K rows per DMA instruction
  constexpr int CPRK = RBK / 16;     // 16-byte chunks per K row
  constexpr int SB = Cfg::SB;
  constexpr int SBK = Cfg::SBK;
  constexpr int NI = SB / 1024 / NW;  // DMA instructions per wave and V block
  static_assert(!F8 || D == 128, "fp8 score product: one 16x16x128 product per tile needs d = 128");
  constexpr int KS = BLK < 64 ? BLK : 64;  // keys per sub-step
  constexpr int NSUB = BLK / KS;
  constexpr int NJT = KS / 16;
  constexpr int NNT = Cfg::NNT;
  constexpr int SLOT = Cfg::SLOT;
  static_assert(NI >= 1 && SB % (1024 * NW) == 0, "whole DMA instructions per wave");
  static_assert(NJT % 2 == 0, "32-key products");

  // K and V stages in separate arrays, so that the compiler can tell the
  // K reads from the V transfers in flight (and the other way round)
  constexpr int NSTG = BAND ? 1 : NS;  // K / V stages (one shared stage with BAND)
  constexpr int KSTEP = BAND ? 1 : NS;  // positions of the column walk per step
  __shared__ __attribute__((aligned(16))) unsigned char Ks[NSTG * SBK];
  __shared__ __attribute__((aligned(16))) unsigned char Vs[NSTG * SB];

  const int tid_all = threadIdx.x;
  const int sg = __builtin_amdgcn_readfirstlane(tid_all / NT);  // key group
  const int tid = tid_all % NT;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int li = lane & 15, g = lane >> 4;
  unsigned char* const Kg = Ks + (BAND ? 0 : sg * SBK);
  unsigned char* const Vg = Vs + (BAND ? 0 : sg * SB);
  // Which block row: with rows of similar length, XCD-aware and grouped by
  // (batch, head), the head's rows longest first (K and V of a head stay in
  // the XCD's L2 while its rows are in flight); otherwise longest first
  // across the whole job, batch index fastest (the long rows start first).
  int z, hr;
  int r0 = 0;          // BAND: the group's first row
  bool row_ok = true;  // BAND: this key group's row is on the grid
  if constexpr (BAND) {
    const int zhn = Z * H;
    r0 = grp[blockIdx.x / zhn];
    z = (blockIdx.x % zhn) % Z;
    const int rr = r0 + sg * stride;
    row_ok = rr < nbr;
    hr = ((blockIdx.x % zhn) / Z) * nbr + (row_ok ? rr : r0);
  } else if (grouped) {
    const int unit = xcd_unit(blockIdx.x, gridDim.x);
    const int zhu = unit / nbr;
    z = zhu / H;
    hr = row_order_h[(zhu % H) * nbr + unit % nbr];
  } else {
    z = blockIdx.x % Z;
    hr = row_order[blockIdx.x / Z];
  }
  const int h = hr / nbr, r = hr % nbr;
  int k0, k1;
  if constexpr (BAND) {
    // the union entries whose columns are on the grid
    auto first_at_least = [&](int v) {
      int lo = 0, hi = nu;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (uoff[mid] < v) lo = mid + 1;
        else hi = mid;
      }
      return lo;
    };
    k0 = first_at_least(-r0);
    k1 = first_at_least(nbc - r0);
  } else {
    k0 = row_ptr[hr];
    k1 = row_ptr[hr + 1];
    // causal: key blocks after the row (wholly above the diagonal) are
    // neither staged nor computed
    if constexpr (CAUSAL) trim_causal<false>(col_idx, r, k0, k1);
  }
  auto col_of = [&](int e) { return BAND ? r0 + uoff[e] : col_idx[e]; };
  const int64_t zh = (int64_t)z * H + h;
  const int64_t Nq = (int64_t)nbr * BLK, Nk = (int64_t)nbc * BLK;
  const int q_lo = r * BLK + wave * 32;  // first query row of this wave
  const unsigned char* Kz = static_cast<const unsigned char*>(Kv) + zh * Nk * RBK;
  const u16* Vz = V + zh * Nk * D;
  // K and V of the (batch, head) as raw buffer resources (the launch checks
  // that each fits in 32-bit offsets): a transfer then takes a scalar base
  // and offset and a 32-bit per-lane offset, with no per-lane 64-bit address
  // arithmetic; reads past the extent would return zeros
  const __amdgpu_buffer_rsrc_t kres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(Kz), 0, (int)(unsigned)(Nk * RBK), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u16*>(Vz), 0, (int)(unsigned)(Nk * RB), kRsrcWord3);

  // ---- Q of both tiles as B fragments (8 values of one row per lane);
  // only the sign of scale*log2(e) is folded in (exact in 16 bits)
  V8 qf[2][NQ];
  i32x8 qf8[2];  // fp8: 32 bytes of one row per lane (d 32 g .. 32 g + 31)
  const float sgn = c > 0.f ? 1.f : (c < 0.f ? -1.f : 0.f);
  const float cs_in = (c == 0.f) ? 1.f : fabsf(c);
  // with dense masks the scores become s * |c| + log2(e) * mask (log2 units)
  const float cs = MASKED ? 1.f : cs_in;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if constexpr (F8) {
      const unsigned char* pq = static_cast<const unsigned char*>(Qv) + (zh * Nq + q_lo + 16 * t + li) * D + 32 * g;
      const i32x4 a = *reinterpret_cast<const i32x4*>(pq), b = *reinterpret_cast<const i32x4*>(pq + 16);
      qf8[t] = i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      if (sgn != 1.f) {  // the sign bit of every byte, or zero (both exact)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf8[t][e] = (sgn < 0.f) ? (qf8[t][e] ^ (int)0x80808080u) : 0;
      }
    } else {
      const u16* pq = static_cast<const u16*>(Qv) + (zh * Nq + q_lo + 16 * t + li) * D + g * 8;
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        qf[t][u] = *reinterpret_cast<const V8*>(pq + u * 32);
        if (sgn != 1.f) {
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[t][u][e] = HT::cvt((float)qf[t][u][e] * sgn);
        }
      }
    }
  }

  // ---- DMA: instruction i of this wave moves rows (wave + NW i) * RPI ..
  // of a block; lane l fills slot l % CPR of row l / CPR with the chunk
  // that the swizzle puts there. The swizzle of a row depends only on the
  // parity of the instruction, so two per-lane offsets cover every one.
  // Byte offsets; rows of RBK bytes (K) use the swizzle of that row size.
  int dofs[2], dofk[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int ri = lane / CPR, slot = lane % CPR;
    dofs[p] = ri * RB + ((slot ^ Swz<D>::f(p * RPI + ri)) * 16);
    const int rk = lane / CPRK, sk = lane % CPRK;
    dofk[p] = rk * RBK + ((sk ^ Swz<RBK / 2>::f(p * RPIK + rk)) * 16);
  }
  const int d_even = (wave & 1) ? dofs[1] : dofs[0];
  const int d_odd = (wave & 1) ? dofs[0] : dofs[1];
  const int dk_even = (wave & 1) ? dofk[1] : dofk[0];
  const int dk_odd = (wave & 1) ? dofk[0] : dofk[1];
  // one part of a matrix: the KS rows of one sub-step (the whole block
  // with one sub-step); NIV (V) and NIK (K) instructions per wave
  constexpr int NIV = NI / NSUB;
  constexpr int NIK = SBK / 1024 / NW / NSUB;
  static_assert(NIK >= 1 && SBK % (1024 * NW * NSUB) == 0, "whole K DMA instructions per wave");

  auto dma_n = [&](__amdgpu_buffer_rsrc_t res, unsigned gofs, unsigned char* spart, int n, int de, int dodd) {
    if constexpr (BAND) {
      // group 0 fills the shared stage (splitting the transfers between
      // the groups measured no faster)
      if (sg != 0) return;
    }
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
      if (i < n) {
        const int I = wave + NW * i;  // uniform
        __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_u8*)(spart + I * 1024), 16,
                                                 (unsigned)(((NW * i) & 1) ? dodd : de), gofs + I * 1024, 0, 0);
      }
    }
  };
  auto dmaK = [&](unsigned gofs, unsigned char* spart) { dma_n(kres, gofs, spart, NIK, dk_even, dk_odd); };
  auto dmaV = [&](unsigned gofs, unsigned char* spart) { dma_n(vres, gofs, spart, NIV, d_even, d_odd); };
  // byte offsets of the KS rows of sub-step x of the block at walk position e
  auto kpart = [&](int e, int x) { return (unsigned)(col_of(e) * BLK + x * KS) * (unsigned)RBK; };
  auto vpart = [&](int e, int x) { return (unsigned)(col_of(e) * BLK + x * KS) * (unsigned)RB; };

  // ---- LDS read offsets (bytes). K: lane (g, li) reads row 16 jt + li,
  // chunk 4u + g; V: lane (g, 4k + m) reads row 4g + k, the 8 bytes at
  // column 16 nt + 4m. Row offsets that are multiples of 16 do not change
  // the swizzle and go into the instruction offsets.
  int koff[NQ], voff[NNT], koff8[2];
#pragma unroll
  for (int u = 0; u < NQ; ++u) koff[u] = li * RBK + (((4 * u + g) ^ Swz<RBK / 2>::f(li)) * 16);
  // fp8: lane (g, li) reads bytes 32 g .. 32 g + 31 of K row 16 jt + li
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) koff8[hh] = li * RBK + (((2 * g + hh) ^ Swz<RBK / 2>::f(li)) * 16);
  {
    const int k = li >> 2, m = li & 3, vr = 4 * g + k;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) voff[nt] = vr * RB + (((2 * nt + (m >> 1)) ^ Swz<D>::f(vr)) * 16) + 8 * (m & 1);
  }

  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  f32x4 o[2][NNT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) o[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const V2 ones = {HT::cvt(1.f), HT::cvt(1.f)};

  // Transfers and barriers. With one sub-step: [A] K of the block has
  // landed -> barrier -> fetch V; score product; softmax; [B] V has landed
  // -> barrier (every wave is past the score product) -> fetch the next K;
  // P.V. With two sub-steps each matrix is moved in halves (the 64 keys of
  // a sub-step, two slots each); without K/V sharing:
  //   K and V of sub-step s have landed -> barrier (every wave is also done
  //   with sub-step s - 1) -> score product on K slot s -> fetch K and V of
  //   sub-step s + 1 into the slots of s - 1 -> softmax -> P.V on V slot s.
  // One barrier per sub-step; it measured 2.3% faster on random_b128_bf16
  // than two (K and V halves in flight in a staggered pipeline, a barrier
  // at each half's landing). With K/V sharing (BAND) the staggered form:
  //   [S x] K half x has landed -> barrier -> score product on K half x
  //         -> fetch the V half that the previous sub-step freed;
  //   [P x] V half x has landed -> barrier -> fetch K half x of the next
  //         block; softmax; P.V on V half x.
  // Every barrier is block-wide (all key groups); transfers complete in
  // issue order, so each wait names how many later ones may stay in flight.
  const int nsteps = (k1 - k0 + KSTEP - 1) / KSTEP;
  const int gofs = BAND ? 0 : sg;  // this group's first position of the walk
  unsigned char* const Kp[2] = {Kg, Kg + KS * RBK};
  unsigned char* const Vp[2] = {Vg, Vg + KS * RB};
  // one barrier per sub-step (two sub-steps, no K/V sharing): K and V of a
  // sub-step are fetched together during the previous one
  constexpr bool ONEBAR = NSUB == 2 && !BAND;
  if (k0 + gofs < k1) {
    dmaK(kpart(k0 + gofs, 0), Kp[0]);
    if constexpr (NSUB == 2) {
      dmaV(vpart(k0 + gofs, 0), Vp[0]);
      if constexpr (!ONEBAR) dmaK(kpart(k0 + gofs, 1), Kp[1]);
    }
  }
  for (int step = 0; step < nsteps; ++step) {
    const int kk = k0 + step * KSTEP + gofs;
    const bool valid = kk < k1;
    const bool has_next = kk + KSTEP < k1;
    const int cb = valid ? col_of(kk) : 0;
    if constexpr (NSUB == 1) {
      wait_vmcnt0();
      __syncthreads();  // [A]
      if (valid) dmaV(vpart(kk, 0), Vp[0]);
    }
    const bool mask_block = CAUSAL && (cb * BLK + BLK - 1 > q_lo);
    // BAND: only the blocks this group's row holds
    const bool mine = !BAND || (row_ok && valid && ((umask[kk] >> sg) & 1));
    const bool compute = valid && mine && !(CAUSAL && cb * BLK > q_lo + 31);

#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const int kofs = sub * KS;
      if constexpr (ONEBAR) {
        // K and V of this sub-step have landed (the only transfers in
        // flight), and every wave is done with the previous sub-step, whose
        // slots the next transfers refill
        wait_vmcnt0();
        lds_barrier();
      } else if constexpr (NSUB == 2) {
        // [S sub]: later transfers in flight: V(this, 0) and K(this, 1)
        // before sub-step 0; V(this, 1) and K(next, 0) before sub-step 1
        if (sub == 0) {
          if (valid) wait_vmcnt<NIK + NIV>(); else wait_vmcnt0();
        } else {
          if (has_next) wait_vmcnt<NIK + NIV>(); else if (valid) wait_vmcnt<NIV>(); else wait_vmcnt0();
        }
        lds_barrier();
      }
      const unsigned char* const Kc = Kp[sub];
      // dense masks of this sub-step, both query tiles (in flight during
      // the score product)
      f32x4 mv[MASKED ? 2 : 1][MASKED ? NJT : 1];
      if constexpr (MASKED) {
        if (compute) {
          const int64_t Nk = (int64_t)nbc * BLK;
          const int64_t key0 = (int64_t)cb * BLK + kofs + 4 * g;
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) {
            // the key-padding values depend on the key only: one read for
            // both query tiles
            f32x4 kpv = {0.f, 0.f, 0.f, 0.f};
            if (kpmask != nullptr) kpv = *reinterpret_cast<const f32x4*>(kpmask + z * Nk + key0 + 16 * jt);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              f32x4 m = kpv;
              if (amask != nullptr)
                m += *reinterpret_cast<const f32x4*>(amask + (int64_t)(q_lo + 16 * t + li) * Nk + key0 + 16 * jt);
              mv[t][jt] = m;
            }
          }
        }
      }
      f32x4 s[2][NJT];
      // ---- S^T = K Q^T for both tiles
      if constexpr (F8) {
        if (compute) {
          // one 16x16x128 fp8 product per key tile and query tile; the K
          // operand (32 bytes a lane) of tile jt+1 is read while tile jt
          // is multiplied
          auto ldk = [&](int jt) {
            const i32x4 a = *reinterpret_cast<const i32x4*>(Kc + 16 * jt * RBK + koff8[0]);
            const i32x4 b = *reinterpret_cast<const i32x4*>(Kc + 16 * jt * RBK + koff8[1]);
            return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
          };
          i32x8 ka8[2];
          ka8[0] = ldk(0);
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) {
            if (jt + 1 < NJT) ka8[(jt + 1) & 1] = ldk(jt + 1);
            __builtin_amdgcn_sched_barrier(0);
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            // format codes 0 (FP8 E4M3) for both operands, no block scales
            s[0][jt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka8[jt & 1], qf8[0], zero, 0, 0, 0, 0, 0, 0);
            s[1][jt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka8[jt & 1], qf8[1], zero, 0, 0, 0, 0, 0, 0);
          }
        }
      } else if (compute) {
        // the K operands of tile jt+1 are read while tile jt is multiplied
        V8 ka[2][NQ];
#pragma unroll
        for (int u = 0; u < NQ; ++u) ka[0][u] = *reinterpret_cast<const V8*>(Kc + koff[u]);
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          if (jt + 1 < NJT) {
#pragma unroll
            for (int u = 0; u < NQ; ++u)
              ka[(jt + 1) & 1][u] = *reinterpret_cast<const V8*>(Kc + 16 * (jt + 1) * RBK + koff[u]);
          }
          __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the products
          s[0][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
          s[1][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < NQ; ++u) {
            s[0][jt] = HT::mfma16(ka[jt & 1][u], qf[0][u], s[0][jt]);
            s[1][jt] = HT::mfma16(ka[jt & 1][u], qf[1][u], s[1][jt]);
          }
        }
      }
      if constexpr (ONEBAR) {
        // the next sub-step's K and V, once this wave's K reads are done
        if (sub == 0) {
          if (valid) {
            dmaK(kpart(kk, 1), Kp[1]);
            dmaV(vpart(kk, 1), Vp[1]);
          }
        } else if (has_next) {
          dmaK(kpart(kk + KSTEP, 0), Kp[0]);
          dmaV(vpart(kk + KSTEP, 0), Vp[0]);
        }
      } else if constexpr (NSUB == 2) {
        // the V half that the previous sub-step freed, issued once this
        // wave's K reads are done: the transfer's LDS writes would
        // otherwise be queued ahead of them (measured 3-5% faster on
        // random_b128_bf16 than issuing it right after the barrier)
        if (sub == 0) {
          if (valid) dmaV(vpart(kk, 1), Vp[1]);
        } else {
          if (has_next) dmaV(vpart(kk + KSTEP, 0), Vp[0]);
        }
        // [P sub]: later transfers in flight: K(this, 1) and V(this, 1)
        // before sub-step 0's P.V; K(next, 0) and V(next, 0) before
        // sub-step 1's
        if (sub == 0) {
          if (valid) wait_vmcnt<NIK + NIV>(); else wait_vmcnt0();
        } else {
          if (has_next) wait_vmcnt<NIK + NIV>(); else wait_vmcnt0();
        }
        lds_barrier();
        if (has_next) dmaK(kpart(kk + KSTEP, sub), Kp[sub]);
      }

      // ---- softmax of both tiles
      if (compute) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int q_index = q_lo + 16 * t + li;
          if constexpr (MASKED) {
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) s[t][jt][rr] = fmaf(mv[t][jt][rr], kLog2eB, s[t][jt][rr] * cs_in);
          }
          if (mask_block) {
#pragma unroll
            for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
              for (int rr = 0; rr < 4; ++rr)
                if (cb * BLK + kofs + 16 * jt + 4 * g + rr > q_index) s[t][jt][rr] = -INFINITY;
          }
          float mx = -INFINITY;
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, s[t][jt][rr]);
          mx = rows4_max(mx);
          const float m_blk = mx * cs;
          const bool upd = m_blk > m_run[t] + kTauB;
          if (__builtin_amdgcn_ballot_w64(upd) != 0) {  // wave-uniform
            const float m_new = upd ? m_blk : m_run[t];
            // 1 for lanes that keep their max (no -inf - -inf); 0 when an
            // update leaves m_run = -inf
            const float alpha = upd ? __builtin_amdgcn_exp2f(m_run[t] - m_new) : 1.f;
            l_run[t] *= alpha;
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) o[t][nt] *= alpha;
            m_run[t] = m_new;
          }
          const float m_sub = (m_run[t] == -INFINITY) ? 0.f : m_run[t];
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) s[t][jt][rr] = __builtin_amdgcn_exp2f(fmaf(s[t][jt][rr], cs, -m_sub));
        }
      }

      if constexpr (NSUB == 1) {
        wait_vmcnt0();    // this wave's part of V (the only transfer in flight)
        __syncthreads();  // [B]
        if (has_next) dmaK(kpart(kk + KSTEP, 0), Kp[0]);
      }
      if (!compute) continue;

      // ---- O^T += V^T P^T for both tiles from one pair of V reads
#pragma unroll
      for (int jp = 0; jp < NJT / 2; ++jp) {
        V8 pb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          pb[t] = V8{HT::cvt(s[t][2 * jp][0]),     HT::cvt(s[t][2 * jp][1]),     HT::cvt(s[t][2 * jp][2]),
                     HT::cvt(s[t][2 * jp][3]),     HT::cvt(s[t][2 * jp + 1][0]), HT::cvt(s[t][2 * jp + 1][1]),
                     HT::cvt(s[t][2 * jp + 1][2]), HT::cvt(s[t][2 * jp + 1][3])};
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            l_run[t] = HT::dot2(V2{pb[t][e], pb[t][e + 1]}, ones, l_run[t]);
        }
        // every V operand of the 32 keys is requested before the first
        // product, so the reads stream behind the MFMAs
        const unsigned char* vb = Vp[sub] + 32 * jp * RB;
        V4 va0[NNT], va1[NNT];
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) {
          va0[nt] = lds_read_tr16_as<V4>(reinterpret_cast<const u16*>(vb + voff[nt]));
          va1[nt] = lds_read_tr16_as<V4>(reinterpret_cast<const u16*>(vb + 16 * RB + voff[nt]));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt) {
          const V8 a = {va0[nt][0], va0[nt][1], va0[nt][2], va0[nt][3],
                            va1[nt][0], va1[nt][1], va1[nt][2], va1[nt][3]};
          o[0][nt] = HT::mfma16(a, pb[0], o[0][nt]);
          o[1][nt] = HT::mfma16(a, pb[1], o[1][nt]);
        }
      }
    }  // sub-step
  }

  // ---- merge the key groups into group 0 through the K stages, one query
  // tile at a time: each side's (l, O) is rescaled by exp2(m_side - m_max)
  if constexpr (BAND) {
    if (!row_ok) return;
  } else if constexpr (NS > 1) {
    float* red = reinterpret_cast<float*>(Ks);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      __syncthreads();
      if (sg > 0) {
        float* slot = red + ((sg - 1) * NW + wave) * SLOT;
        slot[lane] = m_run[t];
        slot[64 + lane] = l_run[t];
#pragma unroll
        for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e) slot[128 + (nt * 4 + e) * 64 + lane] = o[t][nt][e];
      }
      __syncthreads();
      if (sg == 0) {
#pragma unroll
        for (int s2 = 1; s2 < NS; ++s2) {
          const float* slot = red + ((s2 - 1) * NW + wave) * SLOT;
          const float m2 = slot[lane], l2 = slot[64 + lane];
          const float m_new = fmaxf(m_run[t], m2);
          const float a1 = (m_new == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[t] - m_new);
          const float a2 = (m_new == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - m_new);
          l_run[t] = l_run[t] * a1 + l2 * a2;
#pragma unroll
          for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[t][nt][e] = o[t][nt][e] * a1 + slot[128 + (nt * 4 + e) * 64 + lane] * a2;
          m_run[t] = m_new;
        }
      }
    }
    if (sg > 0) return;
  }

  // ---- finish: divide by l (summed over the 4 lane rows), write O rows
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float l = rows4_sum(l_run[t]);
    const float inv = (l > 0.f) ? 1.0f / l : 0.f;
    // row log-sum-exp, natural-log units (l >= 1 when the row saw anything)
    if (lse != nullptr && g == 0)
      lse[zh * Nq + q_lo + 16 * t + li] = (l > 0.f) ? (m_run[t] + __builtin_amdgcn_logf(l)) * kLn2B : -INFINITY;
    u16* po = O + (zh * Nq + q_lo + 16 * t + li) * D + 4 * g;
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt)
      *reinterpret_cast<V4*>(po + nt * 16) =
          V4{HT::cvt(o[t][nt][0] * inv), HT::cvt(o[t][nt][1] * inv), HT::cvt(o[t][nt][2] * inv), HT::cvt(o[t][nt][3] * inv)};
  }
}

template <typename E, int BLK, int D, int NS>
int launch_ns(const bs_layout* L, const AttnArgs& a, float c, hipStream_t s) {
  const void *Q = a.Q, *K = a.K, *V = a.V;
  void* O = a.O;
  const int Z = a.Z;
  const dim3 grid(L->H * L->nbr * Z), block(BLK * 2 * NS);
  // head-grouped order when the longest row (split over NS key groups) is
  // at most a quarter of the work of one workgroup slot (two per CU): then
  // even a long row that starts late adds little to the end of the kernel
  const double per_slot = (double)Z * (double)L->nnz / (2.0 * L->num_cus);
  const int grouped = (4.0 * L->max_row_len / NS <= per_slot) ? 1 : 0;
  const bool masked = a.am != nullptr || a.kp != nullptr;
#define BSA_WIDE_LAUNCH(CA, MA)                                                                                   \
  hipLaunchKernelGGL((k_attn_wide<E, BLK, D, CA, NS, MA>), grid, block, 0, s, L->row_ptr, L->col_idx,            \
                     L->row_order, L->row_order_h, Q, K, (const u16*)V, (u16*)O, Z, L->H,                         \
                     L->nbr, L->nbc, c, grouped, a.lse, a.am, a.kp)
  if (a.causal) {
    if (masked) BSA_WIDE_LAUNCH(true, true);
    else BSA_WIDE_LAUNCH(true, false);
  } else {
    if (masked) BSA_WIDE_LAUNCH(false, true);
    else BSA_WIDE_LAUNCH(false, false);
  }
#undef BSA_WIDE_LAUNCH
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

// K/V shared across two block rows of a slope-1 ACSR layout (its sharing
// plan, when the handle has one and sharing is on; no dense masks)
template <typename E, int BLK, int D>
int launch_band(const bs_layout* L, const AttnArgs& a, float c, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)L->share_ngrp * a.Z * L->H)), block(BLK * 2 * 2);
#define BSA_WIDE_BAND(CA)                                                                                         \
  hipLaunchKernelGGL((k_attn_wide<E, BLK, D, CA, 2, false, true>), grid, block, 0, s, L->row_ptr, L->col_idx,     \
                     L->row_order, L->row_order_h, a.Q, a.K, (const u16*)a.V, (u16*)a.O, a.Z, L->H, L->nbr,       \
                     L->nbc, c, 0, a.lse, nullptr, nullptr, L->share_uoff, L->share_umask, L->share_grp,          \
                     L->share_n, L->share_stride)
  if (a.causal) BSA_WIDE_BAND(true);
  else BSA_WIDE_BAND(false);
#undef BSA_WIDE_BAND
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

// Key groups per workgroup: split a row's blocks over NS groups once the
// longest row alone (about two workgroups share a CU) outlasts a CU's share
// of the job.
template <typename E, int BLK, int D>
int run(const bs_layout* L, const AttnArgs& a, float c, hipStream_t s) {
  const int Z = a.Z;
  // K/V sharing on request, and by default at blocks of 64, where it
  // measured faster on band layouts (strided, 16384 tokens, 16 heads,
  // bf16: d = 128 3%, d = 64 6-7%); at 128-blocks the eight-wave
  // workgroup, one per CU, measured 12-16% slower, at 32-blocks 0-3%
  // faster
  // the transfers address a (batch, head)'s K and V with 32-bit offsets
  if ((int64_t)L->nbc * BLK * 2 * D > 0xFFFFFFFFll) return kNotApplicable;
  if constexpr (!WideTypes<E>::F8) {
    const bool share = L->share_mode == 1 || (L->share_mode == -1 && BLK == 64);
    if (share && L->share_n > 0 && L->share_rows == 2 && a.am == nullptr && a.kp == nullptr)
      return launch_band<E, BLK, D>(L, a, c, s);
  }
  using Cfg = WideCfg<BLK, D, WideTypes<E>::F8 ? D : 2 * D>;
  constexpr size_t cap = 160 * 1024;
  // four groups of a 128-block row would be 1024 threads, at most 128
  // VGPRs a lane, which the causal variant exceeded (it spilled)
  constexpr int max_ns = (Cfg::bytes(4) <= cap && Cfg::merge_fits(4) && BLK * 8 < 1024)
                             ? 4
                             : ((Cfg::bytes(2) <= cap && Cfg::merge_fits(2)) ? 2 : 1);
  const double per_cu = (double)Z * (double)L->nnz / L->num_cus;
  int ns = 1;
  while (ns < max_ns && 2.0 * L->max_row_len / ns > per_cu) ns *= 2;
  if constexpr (max_ns >= 4) {
    if (ns >= 4) return launch_ns<E, BLK, D, 4>(L, a, c, s);
  }
  if constexpr (max_ns >= 2) {
    if (ns >= 2) return launch_ns<E, BLK, D, 2>(L, a, c, s);
  }
  return launch_ns<E, BLK, D, 1>(L, a, c, s);
}

template <typename E, int D>
int run_b(const bs_layout* L, const AttnArgs& a, float c, hipStream_t s) {
  switch (L->block) {
    case 32: return run<E, 32, D>(L, a, c, s);
    case 64: return run<E, 64, D>(L, a, c, s);
    case 128: return run<E, 128, D>(L, a, c, s);
  }
  return kNotApplicable;
}

}  // namespace

int launch_attention_wide(const bs_layout* L, const AttnArgs& a, hipStream_t s) {
  const float c = a.scale * kLog2eB;
  if (a.dt == BS_BF16) {
    if (a.d == 64) return run_b<bf16_t, 64>(L, a, c, s);
    if (a.d == 128) return run_b<bf16_t, 128>(L, a, c, s);
  } else if (a.dt == BS_F16) {
    if (a.d == 64) return run_b<f16_t, 64>(L, a, c, s);
    if (a.d == 128) return run_b<f16_t, 128>(L, a, c, s);
  } else if (a.dt == BS_F8E4M3) {
    // one 16x16x128 fp8 product per tile covers d = 128
    if (a.d == 128) return run_b<f8_t, 128>(L, a, c, s);
  }
  return kNotApplicable;
}

}  // namespace bsa
