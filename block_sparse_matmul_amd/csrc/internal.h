// Internal declarations shared by the C-ABI layer (api.cpp) and the kernel
// translation units. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "bsattn.h"

// Device-resident tables of one layout. One allocation (`mem`) holds every
// array; all are int32.
constexpr int kSoftmaxClasses = 4;  // see softmax_class

struct bs_layout {
  int device = 0;
  int num_cus = 256;  // compute units of the device (scheduling heuristics)
  int H = 0, nbr = 0, nbc = 0, block = 0;
  int64_t nnz = 0;
  int max_row_len = 0;  // longest block row (blocks)
  int max_col_len = 0;  // longest block column (blocks)
  void* mem = nullptr;
  int32_t* row_ptr = nullptr;    // [H*nbr + 1]
  int32_t* col_idx = nullptr;    // [nnz]
  int32_t* col_ptr = nullptr;    // [H*nbc + 1]
  int32_t* row_idx = nullptr;    // [nnz]
  int32_t* blk_id = nullptr;     // [nnz]
  int32_t* row_order = nullptr;  // [H*nbr] block rows, longest first
  int32_t* col_order = nullptr;  // [H*nbc] block columns, longest first
  // the same orders grouped by head: head h's rows at h*nbr.., longest first
  int32_t* row_order_h = nullptr;  // [H*nbr]
  int32_t* col_order_h = nullptr;  // [H*nbc]
  // ACSR layouts whose terms all have slope 1 and cover every row: row r
  // holds the columns r + d for d in this sorted offset set, clipped to the
  // grid (own allocation; null otherwise)
  int32_t* band_off = nullptr;
  int band_n = 0;
  // K/V sharing across block rows on such a layout (attention_band.hip):
  // groups of share_rows rows r0, r0 + share_stride, ...; the group's
  // columns are r0 + share_uoff[i] (ascending), held by the rows whose bits
  // are set in share_umask[i]; share_grp lists every group's r0, longest
  // group first. One allocation (share_mem); share_n = 0 when there is no
  // plan. share_mode: whether the fused attention uses it: 1 yes, 0 no, -1
  // where it measured faster (16-bit operands, blocks of 64).
  int32_t* share_mem = nullptr;
  const int32_t* share_uoff = nullptr;
  const int32_t* share_umask = nullptr;
  const int32_t* share_grp = nullptr;
  int share_n = 0, share_ngrp = 0, share_stride = 0, share_rows = 1;
  int share_mode = -1;
  // non-empty block rows grouped by softmax length class (see
  // softmax_class), class 0 first, (head, row) order inside a class;
  // class c is row_cls[cls_begin[c] .. cls_begin[c+1])
  int32_t* row_cls = nullptr;  // [H*nbr] (in `mem`)
  int cls_begin[kSoftmaxClasses + 1] = {};
  int cls_max_len[kSoftmaxClasses] = {};  // longest row of each class (blocks)
};

// Length class of a block row of `len` blocks of edge b for the row-softmax
// kernels, by the 16-byte vectors per lane a wave keeps of the row (256
// floats per pass): 0 for more than 20 passes, 1 for 17 to 20, 2 for 9 to
// 16, 3 for up to 8.
inline int softmax_class(int64_t len, int b) {
  const int64_t n = len * b;
  return n > 20 * 256 ? 0 : (n > 16 * 256 ? 1 : (n > 8 * 256 ? 2 : 3));
}

// Workgroup -> work unit for kernels that walk a head's rows (or columns)
// together: workgroup b runs on XCD b % 8 (round-robin dispatch), and each
// XCD gets a contiguous range of the G units, so the rows in flight on one
// XCD come from few (batch, head) pairs and share that XCD's L2.
__device__ __forceinline__ int xcd_unit(int b, int G) {
  const int q = G >> 3, rem = G & 7, x = b & 7, j = b >> 3;
  return x * q + (x < rem ? x : rem) + j;
}

// Causal backward walk of block row (DKDV = false) or block column (true) u
// over entries [k0, k1) of an ascending index list: blocks wholly above the
// diagonal (a key block after the row, or a query block before the column)
// have P = 0 and add nothing, and are dropped from the walk. They form a
// tail (rows) or a head (columns) of the list, found by binary search; the
// diagonal block u itself stays.
template <bool DKDV>
__device__ __forceinline__ void trim_causal(const int32_t* __restrict__ idx, int u, int& k0, int& k1) {
  if constexpr (DKDV) {
    if (k0 < k1 && idx[k0] < u) {
      int lo = k0 + 1, hi = k1;  // first entry >= u
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (idx[mid] < u) lo = mid + 1;
        else hi = mid;
      }
      k0 = lo;
    }
  } else {
    if (k0 < k1 && idx[k1 - 1] > u) {
      int lo = k0, hi = k1 - 1;  // first entry > u
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (idx[mid] > u) hi = mid;
        else lo = mid + 1;
      }
      k1 = lo;
    }
  }
}

namespace bsa {

// error reporting (thread-local message, see bs_last_error)
int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* what);

#define BSA_HIP(call)                                   \
  do {                                                  \
    hipError_t e_ = (call);                             \
    if (e_ != hipSuccess) return ::bsa::hip_fail(e_, #call); \
  } while (0)

// ---- LUT builder (lut.hip) ----
// Builds every table of `L` from a device 0/1 layout. L's sizes are set by
// the caller; on success L->mem and the table pointers are set.
int build_tables(bs_layout* L, const uint8_t* layout_dev, hipStream_t s);
// Expands ACSR terms (device array) into a dense device layout.
int expand_acsr(const bs_acsr_term* terms_dev, int n_terms, int H, int nbr,
                int nbc, uint8_t* layout_dev, hipStream_t s);

// ---- operator launchers (one per translation unit) ----
// am, kp: the optional dense additive masks of the softmax and the fused
// attention (float32 [nbr*b][nbc*b] and [Z][nbc*b]; null when absent).
int launch_sdd(const bs_layout* L, const void* A, const void* B, float* S,
               int Z, int K, int trans, bs_dtype dt, hipStream_t s);
int launch_softmax(const bs_layout* L, const float* S, float* P, int Z,
                   float scale, bool causal, const float* am, const float* kp,
                   hipStream_t s);
int launch_dsd(const bs_layout* L, const float* P, const void* B, void* C,
               int Z, int Nd, bs_dtype dt, hipStream_t s);
int launch_dds(const bs_layout* L, const void* A, const float* S, void* C,
               int Z, int M, bs_dtype dt, hipStream_t s);
// Fused attention operands: Q [Z][H][nbr*b][d], K, V [Z][H][nbc*b][d], O
// like Q (dtype dt); optional dense masks am, kp; optional lse, float32
// [Z][H][nbr*b]: the natural-log softmax denominator of every query row
// (-inf where nothing is visible).
struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int Z;
  int d;
  float scale;
  bool causal;
  bs_dtype dt;
  const float* am = nullptr;
  const float* kp = nullptr;
  float* lse = nullptr;
};
int launch_attention(const bs_layout* L, const AttnArgs& a, hipStream_t s);
int launch_softmax_backward(const bs_layout* L, const float* P, const float* dP, float* dS, int Z, float scale,
                            hipStream_t s);
int launch_dsd_t(const bs_layout* L, const float* S, const void* B, void* C, int Z, int Nd, bs_dtype dt,
                 hipStream_t s);

// Fused attention backward (backward.hip): dQ, dK, dV from Q, K, V, the
// forward's O and lse, and dO (all dense operands of dtype dt); Dws: float32
// [Z][H][nbr*b] workspace for D = rowsum(dO * O); optional dense masks.
struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const float* lse;
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  float* Dws;
  int Z;
  int d;
  float scale;
  bool causal;
  bs_dtype dt;
  const float* am = nullptr;
  const float* kp = nullptr;
};
int launch_attention_bwd(const bs_layout* L, const BwdArgs& a, hipStream_t s);
// The fused backward with 32 rows per wave and LDS DMA staging (16-bit
// operands, blocks of 64 or 128, no dense masks); kNotApplicable otherwise.
int launch_attention_bwd_wide(const bs_layout* L, const BwdArgs& a, hipStream_t s);

// The D buffer of bs_attention_bwd_noalloc: float32 [kBwdScratchRows], a
// static device array (backward.hip); *out receives its address on the
// current device (looked up once per device).
constexpr int64_t kBwdScratchRows = (int64_t)1 << 21;  // 8 MiB
int bwd_scratch(float** out);

// DSD and DDS with the BS_TRANS_A / BS_TRANS_B flags (dsd.hip): the plain
// and fast paths where they apply, otherwise the general strided kernel
// (GenArgs: P the block values, B the dense operand, C the output; N the
// output width; TP: walk block columns with the blocks transposed; BT / CT:
// B / C addressed [n][j] instead of [j][n]; ld*: row strides; *_head: the
// (batch, head) strides).
struct GenArgs {
  const float* P;
  const void* B;
  void* C;
  int Z;
  int N;
  bool TP, BT, CT;
  int64_t ldb, b_head, ldc, c_head;
};
int launch_dsd_ex(const bs_layout* L, const float* P, const void* B, void* C, int Z, int Nd, int trans, bs_dtype dt,
                  hipStream_t s);
int launch_dds_ex(const bs_layout* L, const void* A, const float* S, void* C, int Z, int M, int trans, bs_dtype dt,
                  hipStream_t s);

// launch_attention with at least one dense mask (attention_masked.hip)
int launch_attention_masked(const bs_layout* L, const AttnArgs& a, hipStream_t s);

// SDD and DSD on the fused kernel's row-block machinery (LDS-staged
// operands); they apply when the contraction (SDD) or output width (DSD) is
// 64 or 128 and return kNotApplicable otherwise.
constexpr int kNotApplicable = 1;
int launch_sdd_rowblock(const bs_layout* L, const void* A, const void* B,
                        float* S, int Z, int K, bs_dtype dt, hipStream_t s);
int launch_dsd_rowblock(const bs_layout* L, const float* P, const void* B,
                        void* C, int Z, int Nd, bs_dtype dt, hipStream_t s);

// 16-bit (bf16, fp16) fused attention on the 32-rows-per-wave kernel
// (blocks of 32, 64, 128, with or without dense masks); returns
// kNotApplicable for other blocks, head sizes or types.
int launch_attention_wide(const bs_layout* L, const AttnArgs& a, hipStream_t s);
// The fused attention with K/V shared across block rows (float32, a layout
// with a sharing plan, blocks of 32 with d in {64, 128} or 64 with d = 64,
// no dense masks); kNotApplicable otherwise or when sharing is off.
int launch_attention_band(const bs_layout* L, const AttnArgs& a, hipStream_t s);

bool log_enabled();

// Device allocation for the layout tables (the only allocations the library
// makes). With the environment variable BS_FAULT_INJECT=oom it fails the way
// an exhausted device does, without calling hipMalloc: a test hook for the
// BS_ERR_OOM paths, read on every call.
hipError_t dev_alloc(void** p, size_t bytes);
template <typename T>
hipError_t dev_alloc(T** p, size_t bytes) {
  return dev_alloc(reinterpret_cast<void**>(p), bytes);
}

}  // namespace bsa
