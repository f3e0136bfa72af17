// Block-sparse row softmax on SDD output (Triton issue 117, "question on
// blocksparse": it reduces the rows of the SDD output and is the same as
// full-attention softmax; a dense causal mask covers the triangle inside
// diagonal blocks).
//
// For query row i of block row r: x = scale * S over the stored blocks of
// the row, plus the optional dense additive masks (the issue's dense masks:
// am[query][key], shared by batch and heads, and kp[z][key]), causal: -inf
// where key c*b+j > query r*b+i; P = exp(x - max) / sum exp(x - max), zeros
// when nothing is visible. exp is evaluated as exp2(x * log2(e)) on the
// hardware's base-2 exponential (the identity the Triton tutorial's Puzzle 8
// uses), so the masks enter as log2(e) * mask.
//
// One wave per query row; block rows are launched by length class (see
// row_classes). The row's stored entries (len blocks x b floats,
// b contiguous floats per block) are read as 16-byte vectors, 256 floats per
// wave pass, and kept in registers (up to R vectors per lane) between the
// max/sum pass and the write pass, so an in-register row costs one read and
// one write of HBM; longer rows are read a second time. S is read and P
// written with nontemporal (streaming) accesses: each element is touched
// once, so it should not displace cached data. Cross-lane max and sum use
// butterfly shuffles. P may alias S: each vector is read before the same
// lanes write it. exp2 is the hardware v_exp_f32 (results below the
// smallest normal flush to zero).
#include <math.h>

#include "internal.h"
#include "tile.h"

namespace bsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int R, bool CAUSAL>
__global__ __launch_bounds__(256) void k_softmax(const int32_t* __restrict__ row_ptr,
                                                 const int32_t* __restrict__ col_idx,
                                                 const int32_t* __restrict__ rows_sel, const float* S, float* P,
                                                 int rows, int nbr, int b, int64_t nnz, float c,
                                                 const float* __restrict__ am, const float* __restrict__ kp,
                                                 int64_t Nk) {
  const int lane = threadIdx.x & 63;
  const int qrow = blockIdx.x * 4 + (threadIdx.x >> 6);  // (selected block row, i) flattened
  if (qrow >= rows * b) return;
  const int z = blockIdx.y;
  const int lb = __builtin_ctz(b);  // b is a power of two
  const int hr = rows_sel[qrow >> lb], i = qrow & (b - 1);
  const int r = hr % nbr;
  const int k0 = row_ptr[hr], k1 = row_ptr[hr + 1];
  const int n = (k1 - k0) * b;  // stored entries of this row
  const int64_t zbase = (int64_t)z * nnz;
  const int q_index = r * b + i;
  const float NEG = -INFINITY;

  auto addr = [&](int e) -> int64_t {  // element e of the row -> offset in S
    const int kl = e >> lb, j = e & (b - 1);
    return ((zbase + k0 + kl) * b + i) * (int64_t)b + j;
  };
  auto load = [&](int e) -> f32x4 {  // scaled, masked values of entries e..e+3
    f32x4 x = {NEG, NEG, NEG, NEG};
    if (e < n) {
      x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + addr(e)));
      x *= c;
      if (CAUSAL || am != nullptr || kp != nullptr) {
        const int kl = e >> lb, j = e & (b - 1);
        const int key = col_idx[k0 + kl] * b + j;  // 4 consecutive keys in one block
        if (am != nullptr) {
          const f32x4 mv = *reinterpret_cast<const f32x4*>(am + (int64_t)q_index * Nk + key);
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = fmaf(mv[q], kLog2e, x[q]);
        }
        if (kp != nullptr) {
          const f32x4 mv = *reinterpret_cast<const f32x4*>(kp + (int64_t)z * Nk + key);
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = fmaf(mv[q], kLog2e, x[q]);
        }
        if (CAUSAL) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (key + q > q_index) x[q] = NEG;
        }
      }
    }
    return x;
  };

  f32x4 cache[R];
  const int passes = (n + 255) / 256;
  float m = NEG;
#pragma unroll
  for (int p = 0; p < R; ++p) {
    if (p < passes) {
      cache[p] = load(p * 256 + lane * 4);
      m = fmaxf(m, fmaxf(fmaxf(cache[p][0], cache[p][1]), fmaxf(cache[p][2], cache[p][3])));
    }
  }
  for (int p = R; p < passes; ++p) {
    const f32x4 x = load(p * 256 + lane * 4);
    m = fmaxf(m, fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  }
  m = wave_max(m);
  if (m == NEG) {  // nothing visible (empty row, or every entry masked)
    for (int p = 0; p < passes; ++p) {
      const int e = p * 256 + lane * 4;
      if (e < n) *reinterpret_cast<f32x4*>(P + addr(e)) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    return;
  }
  float s = 0.f;
#pragma unroll
  for (int p = 0; p < R; ++p) {
    if (p < passes) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cache[p][q] = __builtin_amdgcn_exp2f(cache[p][q] - m);
        s += cache[p][q];
      }
    }
  }
  for (int p = R; p < passes; ++p) {
    const f32x4 x = load(p * 256 + lane * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) s += __builtin_amdgcn_exp2f(x[q] - m);
  }
  const float inv = 1.0f / wave_sum(s);
#pragma unroll
  for (int p = 0; p < R; ++p) {
    const int e = p * 256 + lane * 4;
    if (p < passes && e < n) __builtin_nontemporal_store(cache[p] * inv, reinterpret_cast<f32x4*>(P + addr(e)));
  }
  for (int p = R; p < passes; ++p) {
    const int e = p * 256 + lane * 4;
    f32x4 x = load(e);
    if (e < n) {
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = __builtin_amdgcn_exp2f(x[q] - m) * inv;
      __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(P + addr(e)));
    }
  }
}

template <int R>
void launch_r(const bs_layout* L, const int32_t* rows_sel, int rows, const float* S, float* P, int Z, float c,
              bool causal, const float* am, const float* kp, hipStream_t s) {
  const dim3 grid((unsigned)(((int64_t)rows * L->block + 3) / 4), Z);
  const int64_t Nk = (int64_t)L->nbc * L->block;
  if (causal)
    hipLaunchKernelGGL((k_softmax<R, true>), grid, dim3(256), 0, s, L->row_ptr, L->col_idx, rows_sel, S, P, rows,
                       L->nbr, L->block, L->nnz, c, am, kp, Nk);
  else
    hipLaunchKernelGGL((k_softmax<R, false>), grid, dim3(256), 0, s, L->row_ptr, L->col_idx, rows_sel, S, P, rows,
                       L->nbr, L->block, L->nnz, c, am, kp, Nk);
}

// Block rows by length class. The number of vectors a wave keeps in
// registers (R) sets the kernel's registers and so its occupancy, and one
// long row would otherwise set R for every row: rows of up to 8 cached
// vectors per lane run at 8 waves per SIMD, 16 and 20 at 4, 32 at 3. Each
// class (softmax_class; a range of the layout's row_cls table) gets its own
// launch, the longest class first. Inside a class the rows keep their
// (head, row) order, which reads S and writes P in address order (measured
// faster than longest first). Rows without blocks are not launched (they
// have nothing to write).
struct RowClass {
  int begin, end, r;  // range in row_cls, cached vectors per lane
};
static int row_classes(const bs_layout* L, RowClass out[kSoftmaxClasses]) {
  // the short class caches 4 vectors when none of its rows needs more
  const int r_short = (int64_t)L->cls_max_len[3] * L->block > 4 * 256 ? 8 : 4;
  const int rs[kSoftmaxClasses] = {32, 20, 16, r_short};
  int n = 0;
  for (int c = 0; c < kSoftmaxClasses; ++c)
    if (L->cls_begin[c + 1] > L->cls_begin[c]) out[n++] = {L->cls_begin[c], L->cls_begin[c + 1], rs[c]};
  return n;
}

// Gradient of the softmax above with respect to its input S, given P and
// dP = dL/dP: per query row D = sum of P * dP over the row's stored entries,
// then dS = scale * P * (dP - D) (entries the mask hid have P = 0 and get
// 0). Same row-per-wave layout; both P and dP are kept in registers (up to R
// vectors each) between the reduction and the write, longer rows are read
// again. dS may alias dP (or P): every vector is read before the same lanes
// write it.
template <int R>
__global__ __launch_bounds__(256) void k_softmax_bwd(const int32_t* __restrict__ row_ptr,
                                                     const int32_t* __restrict__ rows_sel, const float* P,
                                                     const float* dP, float* dS, int rows, int b, int64_t nnz,
                                                     float scale) {
  const int lane = threadIdx.x & 63;
  const int qrow = blockIdx.x * 4 + (threadIdx.x >> 6);  // (selected block row, i) flattened
  if (qrow >= rows * b) return;
  const int z = blockIdx.y;
  const int lb = __builtin_ctz(b);  // b is a power of two
  const int hr = rows_sel[qrow >> lb], i = qrow & (b - 1);
  const int k0 = row_ptr[hr], k1 = row_ptr[hr + 1];
  const int n = (k1 - k0) * b;
  const int64_t zbase = (int64_t)z * nnz;
  auto addr = [&](int e) -> int64_t {
    const int kl = e >> lb, j = e & (b - 1);
    return ((zbase + k0 + kl) * b + i) * (int64_t)b + j;
  };
  auto load = [&](const float* X, int e) -> f32x4 {
    return e < n ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(X + addr(e))) : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  const int passes = (n + 255) / 256;
  // up to 8 cached vectors are loaded unconditionally (zeros past the
  // row's end), which keeps them in fixed registers (measured 3x faster on
  // rows of 32 64-blocks than loading under p < passes); 16 are loaded
  // under the condition (unconditional, the extra registers cost 8%)
  f32x4 cp[R], cd[R];
  float acc = 0.f;
#pragma unroll
  for (int p = 0; p < R; ++p) {
    if (R <= 8 || p < passes) {
      const int e = p * 256 + lane * 4;
      cp[p] = load(P, e);
      cd[p] = load(dP, e);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = fmaf(cp[p][q], cd[p][q], acc);
    }
  }
#pragma unroll 1
  for (int p = R; p < passes; ++p) {
    const int e = p * 256 + lane * 4;
    const f32x4 x = load(P, e), y = load(dP, e);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = fmaf(x[q], y[q], acc);
  }
  const float D = wave_sum(acc);
#pragma unroll
  for (int p = 0; p < R; ++p) {
    const int e = p * 256 + lane * 4;
    if ((R <= 8 || p < passes) && e < n)
      __builtin_nontemporal_store(scale * cp[p] * (cd[p] - D), reinterpret_cast<f32x4*>(dS + addr(e)));
  }
#pragma unroll 1
  for (int p = R; p < passes; ++p) {
    const int e = p * 256 + lane * 4;
    const f32x4 x = load(P, e), y = load(dP, e);
    if (e < n) __builtin_nontemporal_store(scale * x * (y - D), reinterpret_cast<f32x4*>(dS + addr(e)));
  }
}

template <int R>
void launch_bwd_r(const bs_layout* L, const int32_t* rows_sel, int rows, const float* P, const float* dP, float* dS,
                  int Z, float scale, hipStream_t s) {
  const dim3 grid((unsigned)(((int64_t)rows * L->block + 3) / 4), Z);
  hipLaunchKernelGGL((k_softmax_bwd<R>), grid, dim3(256), 0, s, L->row_ptr, rows_sel, P, dP, dS, rows, L->block,
                     L->nnz, scale);
}

}  // namespace

// The gradient caches two vectors (P and dP) per entry, so its longest
// class keeps 16 of each and reads longer rows again.
int launch_softmax_backward(const bs_layout* L, const float* P, const float* dP, float* dS, int Z, float scale,
                            hipStream_t s) {
  RowClass cls[kSoftmaxClasses];
  int n = row_classes(L, cls);
  // at most 16 cached vectors each: adjacent classes (contiguous in row_cls)
  // that end up with the same count share one launch
  int m = 0;
  for (int k = 0; k < n; ++k) {
    cls[k].r = cls[k].r > 16 ? 16 : cls[k].r;
    if (m > 0 && cls[m - 1].r == cls[k].r && cls[m - 1].end == cls[k].begin) cls[m - 1].end = cls[k].end;
    else cls[m++] = cls[k];
  }
  n = m;
  for (int k = 0; k < n; ++k) {
    const int32_t* sel = L->row_cls + cls[k].begin;
    const int rows = cls[k].end - cls[k].begin;
    if (cls[k].r == 4)
      launch_bwd_r<4>(L, sel, rows, P, dP, dS, Z, scale, s);
    else if (cls[k].r == 8)
      launch_bwd_r<8>(L, sel, rows, P, dP, dS, Z, scale, s);
    else
      launch_bwd_r<16>(L, sel, rows, P, dP, dS, Z, scale, s);
  }
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

int launch_softmax(const bs_layout* L, const float* S, float* P, int Z, float scale, bool causal, const float* am,
                   const float* kp, hipStream_t s) {
  const float c = scale * kLog2e;
  RowClass cls[kSoftmaxClasses];
  const int n = row_classes(L, cls);
  for (int k = 0; k < n; ++k) {
    const int32_t* sel = L->row_cls + cls[k].begin;
    const int rows = cls[k].end - cls[k].begin;
    if (cls[k].r == 4)
      launch_r<4>(L, sel, rows, S, P, Z, c, causal, am, kp, s);
    else if (cls[k].r == 8)
      launch_r<8>(L, sel, rows, S, P, Z, c, causal, am, kp, s);
    else if (cls[k].r == 16)
      launch_r<16>(L, sel, rows, S, P, Z, c, causal, am, kp, s);
    else if (cls[k].r == 20)
      launch_r<20>(L, sel, rows, S, P, Z, c, causal, am, kp, s);
    else
      launch_r<32>(L, sel, rows, S, P, Z, c, causal, am, kp, s);
  }
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

}  // namespace bsa
