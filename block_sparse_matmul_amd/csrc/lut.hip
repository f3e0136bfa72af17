// Layout -> lookup tables, built on the GPU.
//
// The layout is a tensor of 0s and 1s with one entry per non-overlapping
// block (Triton issue 117, "question on blocksparse", answer on the layout).
// Stored blocks are numbered in (head, block-row, block-col) order; the
// tables are the block-CSR over rows (row_ptr, col_idx) and the CSC over
// columns (col_ptr, row_idx, blk_id = CSR id of each CSC entry), plus two
// scheduling orders (rows and columns by descending length).
//
// Every table is produced without order-deciding atomics: counts, a
// single-workgroup exclusive scan, then ordered fills (ballot prefix counts
// within a wave for the CSR, an ascending walk per column for the CSC), so
// the result is bit-exact and deterministic. The ACSR expansion (SPLAT
// abstract, affine-compressed rows) evaluates each cell's membership in the
// union of affine terms.
#include <hip/hip_runtime.h>

#include <vector>

#include "internal.h"

namespace bsa {
namespace {

constexpr int kWave = 64;

// summary slots written by the phase-1 kernels
enum { SUM_BAD = 0, SUM_MAXROW = 1, SUM_MAXCOL = 2, SUM_NNZ_ROWS = 3, SUM_NNZ_COLS = 4, SUM_N = 8 };

// One wave per block row: count the ones, flag values other than 0/1.
__global__ __launch_bounds__(256) void k_count_rows(const uint8_t* __restrict__ lay, int rows, int nbc,
                                                    int32_t* __restrict__ count, int32_t* __restrict__ summary) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const uint8_t* p = lay + (int64_t)row * nbc;
  int n = 0, bad = 0;
  for (int c = lane; c < nbc; c += kWave) {
    const uint8_t v = p[c];
    n += (v == 1);
    bad |= (v > 1);
  }
  for (int off = kWave / 2; off > 0; off >>= 1) {
    n += __shfl_xor(n, off);
    bad |= __shfl_xor(bad, off);
  }
  if (lane == 0) {
    count[row] = n;
    if (bad) atomicOr(&summary[SUM_BAD], 1);
    atomicMax(&summary[SUM_MAXROW], n);
  }
}

// One thread per block column (h, c): count the ones down the column.
__global__ __launch_bounds__(256) void k_count_cols(const uint8_t* __restrict__ lay, int H, int nbr, int nbc,
                                                    int32_t* __restrict__ count, int32_t* __restrict__ summary) {
  const int hc = blockIdx.x * blockDim.x + threadIdx.x;
  if (hc >= H * nbc) return;
  const int h = hc / nbc, c = hc % nbc;
  const uint8_t* p = lay + (int64_t)h * nbr * nbc + c;
  int n = 0;
  for (int r = 0; r < nbr; ++r) n += (p[(int64_t)r * nbc] == 1);
  count[hc] = n;
  atomicMax(&summary[SUM_MAXCOL], n);
}

// Exclusive scan of n counts into ptr[0..n] by one workgroup of 1024
// threads: each thread sums a contiguous chunk, the chunk totals are scanned
// in LDS, then each thread writes its chunk. ptr[n] = total.
__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ count, int n, int32_t* __restrict__ ptr,
                                               int32_t* __restrict__ summary, int slot) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += count[i];
  part[t] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 chunk totals
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = (t >= off) ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = part[t] - s;  // exclusive prefix of this chunk
  for (int i = lo; i < hi; ++i) {
    ptr[i] = run;
    run += count[i];
  }
  if (t == 1023) {
    ptr[n] = part[1023];
    summary[slot] = part[1023];
  }
}

// Histogram of lengths (totals do not depend on the order of the adds).
__global__ __launch_bounds__(256) void k_len_hist(const int32_t* __restrict__ count, int n, int32_t* __restrict__ hist) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) atomicAdd(&hist[count[i]], 1);
}

// Stable counting sort by descending length, run by a single wave: bucket
// starts come from a scan over lengths from longest to shortest, then items
// are placed 64 at a time in index order (rank among earlier lanes of the
// same length, counted through LDS).
__global__ __launch_bounds__(64) void k_order(const int32_t* __restrict__ count, int n, int32_t* __restrict__ hist,
                                              int maxlen, int32_t* __restrict__ order) {
  __shared__ int32_t keys[kWave];
  const int lane = threadIdx.x;
  // hist[L] <- number of items longer than L (bucket start), longest first
  int carry = 0;
  for (int base = maxlen; base >= 0; base -= kWave) {
    const int L = base - lane;
    int v = (L >= 0) ? hist[L] : 0;
    // inclusive scan across lanes in lane order
    int inc = v;
    for (int off = 1; off < kWave; off <<= 1) {
      const int u = __shfl_up(inc, off);
      if (lane >= off) inc += u;
    }
    if (L >= 0) hist[L] = carry + inc - v;
    carry += __shfl(inc, kWave - 1);
  }
  __syncthreads();
  for (int base = 0; base < n; base += kWave) {
    const int i = base + lane;
    const int key = (i < n) ? count[i] : -1;
    keys[lane] = key;
    __syncthreads();
    int before = 0, after = 0;
    for (int j = 0; j < kWave; ++j) {
      const int kj = keys[j];
      before += (j < lane && kj == key);
      after += (j > lane && kj == key);
    }
    const int start = (i < n) ? hist[key] : 0;
    __syncthreads();
    if (i < n) {
      order[start + before] = i;
      if (after == 0) hist[key] = start + before + 1;  // last of its length in this chunk
    }
    __syncthreads();
  }
}

// Stable partition of an order by head (item / per_head), run by a single
// wave like the sort above: head h's items land at h*per_head.., in the
// order they have in the input (longest first). cursor[h] counts the items
// of head h placed so far (zero on entry).
__global__ __launch_bounds__(64) void k_group_by_head(const int32_t* __restrict__ in, int n, int per_head,
                                                      int32_t* __restrict__ cursor, int32_t* __restrict__ out) {
  __shared__ int32_t keys[kWave];
  const int lane = threadIdx.x;
  for (int base = 0; base < n; base += kWave) {
    const int i = base + lane;
    const int item = (i < n) ? in[i] : 0;
    const int key = (i < n) ? item / per_head : -1;
    keys[lane] = key;
    __syncthreads();
    int before = 0, after = 0;
    for (int j = 0; j < kWave; ++j) {
      const int kj = keys[j];
      before += (j < lane && kj == key);
      after += (j > lane && kj == key);
    }
    const int start = (i < n) ? cursor[key] : 0;
    __syncthreads();
    if (i < n) {
      out[key * per_head + start + before] = item;
      if (after == 0) cursor[key] = start + before + 1;  // last of its head in this chunk
    }
    __syncthreads();
  }
}

// One wave per block row: write col_idx in ascending column order and the
// id of every stored block into a dense map (read back by the CSC fill).
__global__ __launch_bounds__(256) void k_fill_rows(const uint8_t* __restrict__ lay, int rows, int nbc,
                                                   const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
                                                   int32_t* __restrict__ idmap) {
  const int lane = threadIdx.x & (kWave - 1);
  const int row = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const uint8_t* p = lay + (int64_t)row * nbc;
  int32_t* ids = idmap + (int64_t)row * nbc;
  int pos = row_ptr[row];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int c0 = 0; c0 < nbc; c0 += kWave) {
    const int c = c0 + lane;
    const bool on = (c < nbc) && p[c] == 1;
    const uint64_t mask = __ballot(on);
    if (on) {
      const int at = pos + __popcll(mask & below);
      col_idx[at] = c;
      ids[c] = at;
    }
    pos += __popcll(mask);
  }
}

// One thread per block column: walk rows in ascending order.
__global__ __launch_bounds__(256) void k_fill_cols(const uint8_t* __restrict__ lay, int H, int nbr, int nbc,
                                                   const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ idmap,
                                                   int32_t* __restrict__ row_idx, int32_t* __restrict__ blk_id) {
  const int hc = blockIdx.x * blockDim.x + threadIdx.x;
  if (hc >= H * nbc) return;
  const int h = hc / nbc, c = hc % nbc;
  const int64_t off = (int64_t)h * nbr * nbc + c;
  int pos = col_ptr[hc];
  for (int r = 0; r < nbr; ++r) {
    const int64_t e = off + (int64_t)r * nbc;
    if (lay[e] == 1) {
      row_idx[pos] = r;
      blk_id[pos] = idmap[e];
      ++pos;
    }
  }
}

// ACSR expansion: cell (r, c) is on iff some term holds row r and column
// c = slope*r + offset + stride*k with 0 <= k < count. The same pattern is
// written for every head.
__global__ __launch_bounds__(256) void k_expand_acsr(const bs_acsr_term* __restrict__ terms, int n_terms, int H,
                                                     int nbr, int nbc, uint8_t* __restrict__ lay) {
  const int64_t cell = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (cell >= (int64_t)nbr * nbc) return;
  const int r = (int)(cell / nbc), c = (int)(cell % nbc);
  uint8_t on = 0;
  for (int t = 0; t < n_terms && !on; ++t) {
    const bs_acsr_term tm = terms[t];
    if (r < tm.row_begin || r >= tm.row_end || tm.count <= 0) continue;
    const int64_t d = (int64_t)c - ((int64_t)tm.slope * r + tm.offset);
    if (tm.stride == 0) {
      on = (d == 0);
    } else if (d % tm.stride == 0) {
      const int64_t k = d / tm.stride;
      on = (k >= 0 && k < tm.count);
    }
  }
  for (int h = 0; h < H; ++h) lay[(int64_t)h * nbr * nbc + cell] = on;
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

int expand_acsr(const bs_acsr_term* terms_dev, int n_terms, int H, int nbr, int nbc, uint8_t* layout_dev,
                hipStream_t s) {
  const int64_t cells = (int64_t)nbr * nbc;
  if (cells == 0) return BS_OK;
  hipLaunchKernelGGL(k_expand_acsr, dim3(blocks_for(cells, 256)), dim3(256), 0, s, terms_dev, n_terms, H, nbr, nbc,
                     layout_dev);
  BSA_HIP(hipGetLastError());
  return BS_OK;
}

int build_tables(bs_layout* L, const uint8_t* lay, hipStream_t s) {
  const int H = L->H, nbr = L->nbr, nbc = L->nbc;
  const int rows = H * nbr, cols = H * nbc;
  const int64_t cells = (int64_t)rows * nbc;

  // fixed-size tables: row_ptr, col_ptr, row_order, col_order,
  // row_order_h, col_order_h, row_cls
  const size_t fixed = (size_t)(rows + 1) + (cols + 1) + 3 * (size_t)rows + 2 * (size_t)cols;
  // temporaries: counts, summary, two histograms, two head cursors, id map
  const size_t tmp_n = (size_t)rows + cols + SUM_N + (nbc + 2) + (nbr + 2) + 2 * (size_t)H + (size_t)cells;
  int32_t* fixed_mem = nullptr;
  int32_t* tmp = nullptr;
  if (dev_alloc(&fixed_mem, fixed * sizeof(int32_t)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(BS_ERR_OOM, "device allocation of the layout tables failed");
  }
  if (dev_alloc(&tmp, tmp_n * sizeof(int32_t)) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(fixed_mem);
    return fail(BS_ERR_OOM, "device allocation of the layout build workspace failed");
  }
  int32_t* row_ptr = fixed_mem;
  int32_t* col_ptr = row_ptr + rows + 1;
  int32_t* row_order = col_ptr + cols + 1;
  int32_t* col_order = row_order + rows;
  int32_t* row_order_h = col_order + cols;
  int32_t* col_order_h = row_order_h + rows;
  int32_t* row_cls = col_order_h + cols;
  int32_t* row_cnt = tmp;
  int32_t* col_cnt = row_cnt + rows;
  int32_t* summary = col_cnt + cols;
  int32_t* hist_r = summary + SUM_N;
  int32_t* hist_c = hist_r + (nbc + 2);
  int32_t* cursor_r = hist_c + (nbr + 2);
  int32_t* cursor_c = cursor_r + H;
  int32_t* idmap = cursor_c + H;

  auto cleanup = [&](int code) {
    (void)hipStreamSynchronize(s);
    (void)hipFree(tmp);
    if (code != BS_OK) (void)hipFree(fixed_mem);
    return code;
  };
#define BSA_TRY(call)                                            \
  do {                                                           \
    hipError_t e_ = (call);                                      \
    if (e_ != hipSuccess) return cleanup(hip_fail(e_, #call));   \
  } while (0)

  BSA_TRY(hipMemsetAsync(summary, 0, (SUM_N + (nbc + 2) + (nbr + 2) + 2 * (size_t)H) * sizeof(int32_t), s));
  hipLaunchKernelGGL(k_count_rows, dim3(blocks_for(rows, 4)), dim3(256), 0, s, lay, rows, nbc, row_cnt, summary);
  hipLaunchKernelGGL(k_count_cols, dim3(blocks_for(cols, 256)), dim3(256), 0, s, lay, H, nbr, nbc, col_cnt, summary);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, row_cnt, rows, row_ptr, summary, (int)SUM_NNZ_ROWS);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, col_cnt, cols, col_ptr, summary, (int)SUM_NNZ_COLS);
  hipLaunchKernelGGL(k_len_hist, dim3(blocks_for(rows, 256)), dim3(256), 0, s, row_cnt, rows, hist_r);
  hipLaunchKernelGGL(k_len_hist, dim3(blocks_for(cols, 256)), dim3(256), 0, s, col_cnt, cols, hist_c);
  hipLaunchKernelGGL(k_order, dim3(1), dim3(64), 0, s, row_cnt, rows, hist_r, nbc, row_order);
  hipLaunchKernelGGL(k_order, dim3(1), dim3(64), 0, s, col_cnt, cols, hist_c, nbr, col_order);
  hipLaunchKernelGGL(k_group_by_head, dim3(1), dim3(64), 0, s, row_order, rows, nbr, cursor_r, row_order_h);
  hipLaunchKernelGGL(k_group_by_head, dim3(1), dim3(64), 0, s, col_order, cols, nbc, cursor_c, col_order_h);
  BSA_TRY(hipGetLastError());

  int32_t sum_host[SUM_N];
  std::vector<int32_t> rp_host((size_t)rows + 1);
  BSA_TRY(hipMemcpyAsync(sum_host, summary, sizeof(sum_host), hipMemcpyDeviceToHost, s));
  BSA_TRY(hipMemcpyAsync(rp_host.data(), row_ptr, rp_host.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s));
  BSA_TRY(hipStreamSynchronize(s));
  if (sum_host[SUM_BAD]) return cleanup(fail(BS_ERR_LAYOUT, "layout values must be 0 or 1"));
  if (sum_host[SUM_NNZ_ROWS] != sum_host[SUM_NNZ_COLS])
    return cleanup(fail(BS_ERR_HIP, "internal: row and column block counts differ"));
  const int64_t nnz = sum_host[SUM_NNZ_ROWS];

  // non-empty rows grouped by softmax length class, a stable partition
  std::vector<int32_t> cls_host;
  cls_host.reserve(rows);
  int cls_begin[kSoftmaxClasses + 1] = {}, cls_max_len[kSoftmaxClasses] = {};
  for (int c = 0; c < kSoftmaxClasses; ++c) {
    cls_begin[c] = (int)cls_host.size();
    for (int hr = 0; hr < rows; ++hr) {
      const int len = rp_host[hr + 1] - rp_host[hr];
      if (len > 0 && softmax_class(len, L->block) == c) {
        cls_host.push_back(hr);
        cls_max_len[c] = len > cls_max_len[c] ? len : cls_max_len[c];
      }
    }
  }
  cls_begin[kSoftmaxClasses] = (int)cls_host.size();
  if (!cls_host.empty()) {
    BSA_TRY(hipMemcpyAsync(row_cls, cls_host.data(), cls_host.size() * sizeof(int32_t), hipMemcpyHostToDevice, s));
    BSA_TRY(hipStreamSynchronize(s));
  }

  int32_t* nnz_mem = nullptr;
  if (nnz > 0) {
    if (dev_alloc(&nnz_mem, (size_t)nnz * 3 * sizeof(int32_t)) != hipSuccess) {
      (void)hipGetLastError();
      return cleanup(fail(BS_ERR_OOM, "device allocation of the block tables failed"));
    }
    int32_t* col_idx = nnz_mem;
    int32_t* row_idx = col_idx + nnz;
    int32_t* blk_id = row_idx + nnz;
    hipLaunchKernelGGL(k_fill_rows, dim3(blocks_for(rows, 4)), dim3(256), 0, s, lay, rows, nbc, row_ptr, col_idx,
                       idmap);
    hipLaunchKernelGGL(k_fill_cols, dim3(blocks_for(cols, 256)), dim3(256), 0, s, lay, H, nbr, nbc, col_ptr, idmap,
                       row_idx, blk_id);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      (void)hipFree(nnz_mem);
      return cleanup(hip_fail(e, "layout table fill"));
    }
    L->col_idx = col_idx;
    L->row_idx = row_idx;
    L->blk_id = blk_id;
  }
#undef BSA_TRY
  cleanup(BS_OK);
  L->nnz = nnz;
  L->max_row_len = sum_host[SUM_MAXROW];
  L->max_col_len = sum_host[SUM_MAXCOL];
  L->row_cls = row_cls;
  for (int c = 0; c <= kSoftmaxClasses; ++c) L->cls_begin[c] = cls_begin[c];
  for (int c = 0; c < kSoftmaxClasses; ++c) L->cls_max_len[c] = cls_max_len[c];
  L->mem = fixed_mem;
  L->row_ptr = row_ptr;
  L->col_ptr = col_ptr;
  L->row_order = row_order;
  L->col_order = col_order;
  L->row_order_h = row_order_h;
  L->col_order_h = col_order_h;
  // the nnz arrays live in their own allocation, remembered through col_idx
  return BS_OK;
}

}  // namespace bsa
