// C-ABI entry points: argument validation (before any HIP call), handle
// management, and dispatch to the kernel launchers. The operations and their
// meaning are documented in include/bsattn.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <limits>
#include <string>

#include <algorithm>
#include <vector>

#include "internal.h"

namespace bsa {

static thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  if (log_enabled()) fprintf(stderr, "[bsattn] error %d: %s\n", code, msg.c_str());
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  const bool oom = (e == hipErrorOutOfMemory);
  return fail(oom ? BS_ERR_OOM : BS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

hipError_t dev_alloc(void** p, size_t bytes) {
  const char* v = getenv("BS_FAULT_INJECT");
  if (v && std::string(v) == "oom") {
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  return hipMalloc(p, bytes);
}

bool log_enabled() {
  static const bool on = [] {
    const char* v = getenv("BS_LOG");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

}  // namespace bsa

using bsa::fail;

namespace {

bool block_ok(int b) { return b == 16 || b == 32 || b == 64 || b == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_handle(bs_layout_t L) {
  if (!L) return fail(BS_ERR_INVALID_ARG, "layout handle is NULL");
  return BS_OK;
}

int check_dims(int H, int nbr, int nbc, int block) {
  if (!block_ok(block)) return fail(BS_ERR_UNSUPPORTED, "block must be 16, 32, 64 or 128");
  if (H <= 0 || nbr <= 0 || nbc <= 0) return fail(BS_ERR_INVALID_ARG, "H, nbr and nbc must be positive");
  const int64_t cells = (int64_t)H * nbr * nbc;
  if (cells > std::numeric_limits<int32_t>::max() || (int64_t)nbr * block > std::numeric_limits<int32_t>::max() ||
      (int64_t)nbc * block > std::numeric_limits<int32_t>::max())
    return fail(BS_ERR_SHAPE, "layout too large for 32-bit block indices");
  return BS_OK;
}

// one workgroup per (batch, block row / column) on a 1-D grid
int check_grid(const bs_layout* L, int Z) {
  const int64_t units = (int64_t)Z * L->H * (L->nbr > L->nbc ? L->nbr : L->nbc);
  // below 2^22 workgroups: with up to 1024 threads each, the grid stays under 2^32 work-items
  if (units >= (int64_t)1 << 22) return fail(BS_ERR_SHAPE, "Z*H*blocks per side must be below 2^22 workgroups");
  return BS_OK;
}

// the dense masks are read as 16-byte vectors
int check_masks(const float* attn_mask, const float* kp_mask) {
  if ((reinterpret_cast<uintptr_t>(attn_mask) & 15) || (reinterpret_cast<uintptr_t>(kp_mask) & 15))
    return fail(BS_ERR_INVALID_ARG, "mask pointers must be 16-byte aligned");
  return BS_OK;
}

int check_dtype(bs_dtype dt, bool fused_attention = false) {
  if (dt == BS_F8E4M3) {
    if (!fused_attention) return fail(BS_ERR_UNSUPPORTED, "BS_F8E4M3 is supported by the fused attention only");
    return BS_OK;
  }
  if (dt != BS_F32 && dt != BS_BF16 && dt != BS_F16)
    return fail(BS_ERR_INVALID_ARG, "dtype must be BS_F32, BS_BF16, BS_F16 or BS_F8E4M3");
  return BS_OK;
}

int current_device_ok() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n == 0) {
    (void)hipGetLastError();
    return fail(BS_ERR_NO_DEVICE, "no HIP device is visible");
  }
  return BS_OK;
}

// Tensor pointers used by a compute call: non-NULL and 16-byte aligned
// whenever there is work to do.
int check_ptrs(bool work, std::initializer_list<const void*> ptrs) {
  if (!work) return BS_OK;
  for (const void* p : ptrs) {
    if (!p) return fail(BS_ERR_INVALID_ARG, "tensor pointer is NULL");
    if (!aligned16(p)) return fail(BS_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  }
  return BS_OK;
}

void log_call(const char* name, const bs_layout* L, int Z, int x) {
  if (bsa::log_enabled())
    fprintf(stderr, "[bsattn] %s H=%d nbr=%d nbc=%d b=%d nnz=%lld Z=%d dim=%d\n", name, L->H, L->nbr, L->nbc,
            L->block, (long long)L->nnz, Z, x);
}

int finish_build(bs_layout* L, const uint8_t* layout, hipStream_t s, bs_layout_t* out) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, L->device) == hipSuccess && cus > 0)
    L->num_cus = cus;
  else
    (void)hipGetLastError();
  const int rc = bsa::build_tables(L, layout, s);
  if (rc != BS_OK) {
    delete L;
    return rc;
  }
  *out = L;
  return BS_OK;
}

}  // namespace

extern "C" {

int bs_version(void) { return 100; }

const char* bs_last_error(void) { return bsa::g_last_error.c_str(); }

int bs_layout_build(const uint8_t* layout, int H, int nbr, int nbc, int block, void* stream, bs_layout_t* out) {
  if (!out) return fail(BS_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int rc = check_dims(H, nbr, nbc, block);
  if (rc) return rc;
  if (!layout) return fail(BS_ERR_INVALID_ARG, "layout pointer is NULL");
  if ((rc = current_device_ok())) return rc;
  bs_layout* L = new bs_layout();
  L->H = H;
  L->nbr = nbr;
  L->nbc = nbc;
  L->block = block;
  if (hipGetDevice(&L->device) != hipSuccess) {
    delete L;
    return fail(BS_ERR_HIP, "hipGetDevice failed");
  }
  if (bsa::log_enabled()) fprintf(stderr, "[bsattn] layout_build H=%d nbr=%d nbc=%d b=%d\n", H, nbr, nbc, block);
  return finish_build(L, layout, (hipStream_t)stream, out);
}

// K/V sharing plan for a slope-1 ACSR layout with offset set d (sorted):
// the fused attention kernels that share K/V (attention_band.hip for
// float32, blocks of 32 and 64; the BAND mode of attention_wide.hip for
// 16-bit operands, blocks of 32 to 128) run G = 2 block rows per
// workgroup, rows r0, r0 + t, ..., r0 + (G-1) t, and stage the union of
// their columns once. The row stride t (1..64, with G rows on
// the grid) is the one whose union U of d, d + t, ..., d + (G-1) t is
// smallest; the plan is kept when U is at most two thirds of the G |d|
// blocks the rows hold between them. Groups: for each residue of r0 mod t,
// runs of G rows of that residue; listed longest first (blocks of U on the
// grid that a row of the group holds), ties by r0.
static int plan_share(bs_layout* L, const std::vector<int32_t>& d) {
  if (L->block < 32 || L->nbr < 2 || d.empty()) return BS_OK;
  constexpr int G = 2;
  const int tmax = std::min(64, (L->nbr - 1) / (G - 1));
  int best_t = 0;
  std::vector<std::pair<int32_t, int32_t>> best;  // (offset, row mask), ascending
  for (int t = 1; t <= tmax; ++t) {
    std::vector<std::pair<int32_t, int32_t>> u;
    u.reserve(d.size() * G);
    for (int jj = 0; jj < G; ++jj)
      for (int32_t o : d) u.emplace_back(o + jj * t, 1 << jj);
    std::sort(u.begin(), u.end());
    std::vector<std::pair<int32_t, int32_t>> m;  // merge equal offsets
    for (const auto& e : u) {
      if (!m.empty() && m.back().first == e.first) m.back().second |= e.second;
      else m.push_back(e);
    }
    if (best_t == 0 || m.size() < best.size()) {
      best_t = t;
      best = std::move(m);
    }
  }
  if (best_t == 0 || 3 * best.size() > 2 * (size_t)G * d.size()) return BS_OK;
  const int t = best_t;
  std::vector<std::pair<int64_t, int32_t>> groups;  // (-length, r0)
  for (int rho = 0; rho < t && rho < L->nbr; ++rho) {
    for (int r0 = rho; r0 < L->nbr; r0 += G * t) {
      int vm = 0;
      for (int jj = 0; jj < G; ++jj)
        if (r0 + jj * t < L->nbr) vm |= 1 << jj;
      int64_t len = 0;
      for (const auto& e : best)
        if (r0 + e.first >= 0 && r0 + e.first < L->nbc && (e.second & vm)) ++len;
      groups.emplace_back(-len, r0);
    }
  }
  std::sort(groups.begin(), groups.end());
  const size_t n = best.size(), ng = groups.size();
  std::vector<int32_t> host(2 * n + ng);
  for (size_t i = 0; i < n; ++i) {
    host[i] = best[i].first;
    host[n + i] = best[i].second;
  }
  for (size_t i = 0; i < ng; ++i) host[2 * n + i] = groups[i].second;
  int32_t* dev = nullptr;
  if (bsa::dev_alloc(&dev, host.size() * sizeof(int32_t)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(BS_ERR_OOM, "device allocation of the K/V sharing plan failed");
  }
  hipError_t e = hipMemcpy(dev, host.data(), host.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(dev);
    return bsa::hip_fail(e, "hipMemcpy(K/V sharing plan)");
  }
  L->share_mem = dev;
  L->share_uoff = dev;
  L->share_umask = dev + n;
  L->share_grp = dev + 2 * n;
  L->share_n = (int)n;
  L->share_ngrp = (int)ng;
  L->share_stride = t;
  L->share_rows = G;
  return BS_OK;
}

// ACSR terms analysed on the host (SPLAT's just-in-time reading of the
// format): when every term has slope 1 and covers every row, the columns of
// row r are r + d for d in one set of relative offsets (the union of the
// terms' offset + stride*k), clipped to the grid. That set, sorted, lets the
// fused kernel compute a row's columns instead of loading them. Offsets that
// no row can use (outside -(nbr-1) .. nbc-1) are dropped. Returns BS_OK also
// when the terms do not qualify (the handle then keeps only the CSR tables).
static int analyse_band(bs_layout* L, const bs_acsr_term* terms, int n_terms) {
  if (n_terms == 0) return BS_OK;
  const int64_t lo = -(int64_t)(L->nbr - 1), hi = (int64_t)L->nbc - 1;
  std::vector<int32_t> d;
  for (int t = 0; t < n_terms; ++t) {
    const bs_acsr_term& T = terms[t];
    if (T.slope != 1 || T.row_begin > 0 || T.row_end < L->nbr) return BS_OK;
    if ((int64_t)T.count > 2 * (hi - lo + 1)) return BS_OK;  // beyond any row: leave it to the tables
    for (int64_t k = 0; k < T.count; ++k) {
      const int64_t v = (int64_t)T.offset + (int64_t)T.stride * k;
      if (v >= lo && v <= hi) d.push_back((int32_t)v);
    }
  }
  std::sort(d.begin(), d.end());
  d.erase(std::unique(d.begin(), d.end()), d.end());
  if (d.empty()) return BS_OK;
  int32_t* dev = nullptr;
  if (bsa::dev_alloc(&dev, d.size() * sizeof(int32_t)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(BS_ERR_OOM, "device allocation of the ACSR offsets failed");
  }
  hipError_t e = hipMemcpy(dev, d.data(), d.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(dev);
    return bsa::hip_fail(e, "hipMemcpy(ACSR offsets)");
  }
  L->band_off = dev;
  L->band_n = (int)d.size();
  return plan_share(L, d);
}

int bs_layout_build_acsr(const bs_acsr_term* terms, int n_terms, int H, int nbr, int nbc, int block, void* stream,
                         bs_layout_t* out) {
  if (!out) return fail(BS_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  int rc = check_dims(H, nbr, nbc, block);
  if (rc) return rc;
  if (n_terms < 0 || (n_terms > 0 && !terms)) return fail(BS_ERR_INVALID_ARG, "terms pointer is NULL");
  for (int t = 0; t < n_terms; ++t) {
    if (terms[t].row_begin > terms[t].row_end || terms[t].count < 0)
      return fail(BS_ERR_INVALID_ARG, "ACSR term needs row_begin <= row_end and count >= 0");
  }
  if ((rc = current_device_ok())) return rc;
  hipStream_t s = (hipStream_t)stream;
  const size_t cells = (size_t)H * nbr * nbc;
  uint8_t* lay = nullptr;
  bs_acsr_term* dterms = nullptr;
  if (bsa::dev_alloc(&lay, cells) != hipSuccess) {
    (void)hipGetLastError();
    return fail(BS_ERR_OOM, "device allocation of the expanded layout failed");
  }
  if (n_terms > 0 && bsa::dev_alloc(&dterms, sizeof(bs_acsr_term) * n_terms) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(lay);
    return fail(BS_ERR_OOM, "device allocation of the ACSR terms failed");
  }
  hipError_t e = hipSuccess;
  if (n_terms > 0)
    e = hipMemcpyAsync(dterms, terms, sizeof(bs_acsr_term) * n_terms, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) rc = bsa::expand_acsr(dterms, n_terms, H, nbr, nbc, lay, s);
  else rc = bsa::hip_fail(e, "hipMemcpyAsync(ACSR terms)");
  if (rc == BS_OK) {
    bs_layout* L = new bs_layout();
    L->H = H;
    L->nbr = nbr;
    L->nbc = nbc;
    L->block = block;
    (void)hipGetDevice(&L->device);
    rc = finish_build(L, lay, s, out);  // synchronises s before returning
    if (rc == BS_OK && (rc = analyse_band(*out, terms, n_terms)) != BS_OK) {
      bs_layout_free(*out);
      *out = nullptr;
    }
  } else {
    (void)hipStreamSynchronize(s);
  }
  (void)hipFree(dterms);
  (void)hipFree(lay);
  return rc;
}

int bs_layout_nnz(bs_layout_t L, int64_t* nnz) {
  if (int rc = check_handle(L)) return rc;
  if (!nnz) return fail(BS_ERR_INVALID_ARG, "nnz pointer is NULL");
  *nnz = L->nnz;
  return BS_OK;
}

int bs_layout_kv_share(bs_layout_t L, int* rows, int* stride) {
  if (int rc = check_handle(L)) return rc;
  if (!rows || !stride) return fail(BS_ERR_INVALID_ARG, "rows or stride pointer is NULL");
  *rows = L->share_n > 0 ? L->share_rows : 1;
  *stride = L->share_n > 0 ? L->share_stride : 0;
  return BS_OK;
}

int bs_layout_set_kv_share(bs_layout_t L, int mode) {
  if (int rc = check_handle(L)) return rc;
  if (mode < -1 || mode > 1) return fail(BS_ERR_INVALID_ARG, "mode must be -1, 0 or 1");
  L->share_mode = mode;
  return BS_OK;
}

int bs_layout_info(bs_layout_t L, int* H, int* nbr, int* nbc, int* block, int64_t* nnz) {
  if (int rc = check_handle(L)) return rc;
  if (H) *H = L->H;
  if (nbr) *nbr = L->nbr;
  if (nbc) *nbc = L->nbc;
  if (block) *block = L->block;
  if (nnz) *nnz = L->nnz;
  return BS_OK;
}

int bs_layout_export(bs_layout_t L, int32_t* row_ptr, int32_t* col_idx, int32_t* col_ptr, int32_t* row_idx,
                     int32_t* blk_id) {
  if (int rc = check_handle(L)) return rc;
  struct Item {
    int32_t* dst;
    const int32_t* src;
    int64_t n;
  } items[] = {{row_ptr, L->row_ptr, (int64_t)L->H * L->nbr + 1},
               {col_idx, L->col_idx, L->nnz},
               {col_ptr, L->col_ptr, (int64_t)L->H * L->nbc + 1},
               {row_idx, L->row_idx, L->nnz},
               {blk_id, L->blk_id, L->nnz}};
  for (const Item& it : items) {
    if (!it.dst || it.n == 0) continue;
    BSA_HIP(hipMemcpy(it.dst, it.src, sizeof(int32_t) * it.n, hipMemcpyDeviceToHost));
  }
  return BS_OK;
}

void bs_layout_free(bs_layout_t L) {
  if (!L) return;
  if (L->col_idx) (void)hipFree(L->col_idx);  // start of the nnz allocation
  if (L->mem) (void)hipFree(L->mem);
  if (L->band_off) (void)hipFree(L->band_off);
  if (L->share_mem) (void)hipFree(L->share_mem);
  delete L;
}

int bs_sdd(bs_layout_t L, const void* A, const void* B, float* S, int Z, int K, bs_dtype dt, void* stream) {
  return bs_sdd_ex(L, A, B, S, Z, K, 0, dt, stream);
}

int bs_sdd_ex(bs_layout_t L, const void* A, const void* B, float* S, int Z, int K, int trans, bs_dtype dt,
              void* stream) {
  if (int rc = check_handle(L)) return rc;
  if (trans & ~(BS_TRANS_A | BS_TRANS_B)) return fail(BS_ERR_INVALID_ARG, "unknown transpose flag");
  if (int rc = check_dtype(dt)) return rc;
  if (Z < 0 || K <= 0) return fail(BS_ERR_INVALID_ARG, "Z must be >= 0 and K > 0");
  if (K % 16) return fail(BS_ERR_UNSUPPORTED, "K must be a multiple of 16");
  const bool work = Z > 0 && L->nnz > 0;
  if (int rc = check_ptrs(work, {A, B, S})) return rc;
  if (!work) return BS_OK;
  if (int rc = check_grid(L, Z)) return rc;
  if ((int64_t)Z * L->nnz * L->block * L->block > ((int64_t)1 << 46))
    return fail(BS_ERR_SHAPE, "block-sparse tensor too large");
  log_call("sdd", L, Z, K);
  return bsa::launch_sdd(L, A, B, S, Z, K, trans, dt, (hipStream_t)stream);
}

int bs_softmax(bs_layout_t L, const float* S, float* P, int Z, float scale, int flags, void* stream) {
  return bs_softmax_masked(L, S, P, Z, scale, flags, nullptr, nullptr, stream);
}

int bs_softmax_masked(bs_layout_t L, const float* S, float* P, int Z, float scale, int flags, const float* attn_mask,
                      const float* kp_mask, void* stream) {
  if (int rc = check_handle(L)) return rc;
  if (int rc = check_masks(attn_mask, kp_mask)) return rc;
  if (flags & ~BS_CAUSAL) return fail(BS_ERR_INVALID_ARG, "unknown flag");
  if (Z < 0) return fail(BS_ERR_INVALID_ARG, "Z must be >= 0");
  const bool causal = flags & BS_CAUSAL;
  if (causal && L->nbr != L->nbc) return fail(BS_ERR_INVALID_ARG, "causal softmax needs a square layout");
  const bool work = Z > 0 && L->nnz > 0;
  if (int rc = check_ptrs(work, {S, P})) return rc;
  if (!work) return BS_OK;
  if ((int64_t)L->H * L->nbr * L->block > std::numeric_limits<int32_t>::max() - 4)
    return fail(BS_ERR_SHAPE, "too many query rows");
  log_call("softmax", L, Z, flags);
  return bsa::launch_softmax(L, S, P, Z, scale, causal, attn_mask, kp_mask, (hipStream_t)stream);
}

int bs_dsd(bs_layout_t L, const float* P, const void* B, void* C, int Z, int Nd, bs_dtype dt, void* stream) {
  return bs_dsd_ex(L, P, B, C, Z, Nd, 0, dt, stream);
}

int bs_dsd_ex(bs_layout_t L, const float* P, const void* B, void* C, int Z, int Nd, int trans, bs_dtype dt,
              void* stream) {
  if (int rc = check_handle(L)) return rc;
  if (trans & ~(BS_TRANS_A | BS_TRANS_B)) return fail(BS_ERR_INVALID_ARG, "unknown transpose flag");
  if (int rc = check_dtype(dt)) return rc;
  if (Z < 0 || Nd <= 0) return fail(BS_ERR_INVALID_ARG, "Z must be >= 0 and Nd > 0");
  if (Nd % 16) return fail(BS_ERR_UNSUPPORTED, "Nd must be a multiple of 16");
  const bool work = Z > 0;
  if (int rc = check_ptrs(work, {B, C})) return rc;
  if (work && L->nnz > 0) {
    if (int rc = check_ptrs(true, {P})) return rc;
  }
  if (!work) return BS_OK;
  if (int rc = check_grid(L, Z)) return rc;
  log_call("dsd", L, Z, Nd);
  return bsa::launch_dsd_ex(L, P, B, C, Z, Nd, trans, dt, (hipStream_t)stream);
}

int bs_softmax_backward(bs_layout_t L, const float* P, const float* dP, float* dS, int Z, float scale, void* stream) {
  if (int rc = check_handle(L)) return rc;
  if (Z < 0) return fail(BS_ERR_INVALID_ARG, "Z must be >= 0");
  const bool work = Z > 0 && L->nnz > 0;
  if (int rc = check_ptrs(work, {P, dP, dS})) return rc;
  if (!work) return BS_OK;
  if ((int64_t)L->H * L->nbr * L->block > std::numeric_limits<int32_t>::max() - 4)
    return fail(BS_ERR_SHAPE, "too many query rows");
  log_call("softmax_backward", L, Z, 0);
  return bsa::launch_softmax_backward(L, P, dP, dS, Z, scale, (hipStream_t)stream);
}

int bs_dsd_t(bs_layout_t L, const float* S, const void* B, void* C, int Z, int Nd, bs_dtype dt, void* stream) {
  if (int rc = check_handle(L)) return rc;
  if (int rc = check_dtype(dt)) return rc;
  if (Z < 0 || Nd <= 0) return fail(BS_ERR_INVALID_ARG, "Z must be >= 0 and Nd > 0");
  if (Nd != 64 && Nd != 128) return fail(BS_ERR_UNSUPPORTED, "Nd must be 64 or 128");
  const bool work = Z > 0;
  if (int rc = check_ptrs(work, {B, C})) return rc;
  if (work && L->nnz > 0) {
    if (int rc = check_ptrs(true, {S})) return rc;
  }
  if (!work) return BS_OK;
  if (int rc = check_grid(L, Z)) return rc;
  log_call("dsd_t", L, Z, Nd);
  return bsa::launch_dsd_t(L, S, B, C, Z, Nd, dt, (hipStream_t)stream);
}

int bs_attention_backward(bs_layout_t L, const void* Q, const void* K, const void* V, const void* dO, void* dQ,
                          void* dK, void* dV, float* ws_s, float* ws_p, int Z, int d, float scale, int flags,
                          bs_dtype dt, void* stream) {
  return bs_attention_backward_masked(L, Q, K, V, dO, dQ, dK, dV, ws_s, ws_p, Z, d, scale, flags, nullptr, nullptr,
                                      dt, stream);
}

int bs_attention_backward_masked(bs_layout_t L, const void* Q, const void* K, const void* V, const void* dO,
                                 void* dQ, void* dK, void* dV, float* ws_s, float* ws_p, int Z, int d, float scale,
                                 int flags, const float* attn_mask, const float* kp_mask, bs_dtype dt,
                                 void* stream) {
  if (int rc = check_handle(L)) return rc;
  if (int rc = check_masks(attn_mask, kp_mask)) return rc;
  if (int rc = check_dtype(dt)) return rc;
  if (flags & ~BS_CAUSAL) return fail(BS_ERR_INVALID_ARG, "unknown flag");
  if (Z < 0) return fail(BS_ERR_INVALID_ARG, "Z must be >= 0");
  if (d != 64 && d != 128) return fail(BS_ERR_UNSUPPORTED, "head size d must be 64 or 128");
  const bool causal = flags & BS_CAUSAL;
  if (causal && L->nbr != L->nbc) return fail(BS_ERR_INVALID_ARG, "causal attention needs a square layout");
  const bool work = Z > 0;
  if (int rc = check_ptrs(work, {Q, K, V, dO, dQ, dK, dV})) return rc;
  if (work && L->nnz > 0) {
    if (int rc = check_ptrs(true, {ws_s, ws_p})) return rc;
  }
  if (!work) return BS_OK;
  if (int rc = check_grid(L, Z)) return rc;
  if ((int64_t)Z * L->nnz * L->block * L->block > ((int64_t)1 << 46))
    return fail(BS_ERR_SHAPE, "block-sparse tensor too large");
  if ((int64_t)L->H * L->nbr * L->block > std::numeric_limits<int32_t>::max() - 4)
    return fail(BS_ERR_SHAPE, "too many query rows");
  log_call("attention_backward", L, Z, d);
  hipStream_t s = (hipStream_t)stream;
  if (int rc = bsa::launch_sdd(L, Q, K, ws_s, Z, d, 0, dt, s)) return rc;               // S = Q K^T
  if (int rc = bsa::launch_softmax(L, ws_s, ws_p, Z, scale, causal, attn_mask, kp_mask, s)) return rc;  // P
  if (int rc = bsa::launch_sdd(L, dO, V, ws_s, Z, d, 0, dt, s)) return rc;              // dP = dO V^T
  if (int rc = bsa::launch_softmax_backward(L, ws_p, ws_s, ws_s, Z, scale, s)) return rc;  // dS
  if (int rc = bsa::launch_dsd(L, ws_s, K, dQ, Z, d, dt, s)) return rc;                 // dQ = dS K
  if (int rc = bsa::launch_dsd_t(L, ws_s, Q, dK, Z, d, dt, s)) return rc;               // dK = dS^T Q
  return bsa::launch_dsd_t(L, ws_p, dO, dV, Z, d, dt, s);                               // dV = P^T dO
}

}  // extern "C"

// Shared body of bs_attention_bwd (D in the caller's ws_d) and
// bs_attention_bwd_noalloc (D in the library's static device array, no
// allocation of any kind).
static int attention_bwd(bs_layout_t L, const void* Q, const void* K, const void* V, const void* O, const float* lse,
                         const void* dO, void* dQ, void* dK, void* dV, float* ws_d, bool use_scratch, int Z, int d,
                         float scale, int flags, const float* attn_mask, const float* kp_mask, bs_dtype dt,
                         void* stream) {
  if (int rc = check_handle(L)) return rc;
  if (use_scratch && Z > 0 && (int64_t)Z * L->H * L->nbr * L->block > bsa::kBwdScratchRows)
    return fail(BS_ERR_SHAPE, "bs_attention_bwd_noalloc: Z*H*nbr*b = " +
                                  std::to_string((int64_t)Z * L->H * L->nbr * L->block) +
                                  " query rows exceed the static D buffer of " +
                                  std::to_string(bsa::kBwdScratchRows) + " rows (use bs_attention_bwd)");
  if (int rc = check_dtype(dt)) return rc;
  if (int rc = check_masks(attn_mask, kp_mask)) return rc;
  if (flags & ~BS_CAUSAL) return fail(BS_ERR_INVALID_ARG, "unknown flag");
  if (Z < 0) return fail(BS_ERR_INVALID_ARG, "Z must be >= 0");
  if (d != 64 && d != 128) return fail(BS_ERR_UNSUPPORTED, "head size d must be 64 or 128");
  const bool causal = flags & BS_CAUSAL;
  if (causal && L->nbr != L->nbc) return fail(BS_ERR_INVALID_ARG, "causal attention needs a square layout");
  const bool work = Z > 0;
  if (int rc = check_ptrs(work, {Q, K, V, O, lse, dO, dQ, dK, dV})) return rc;
  if (!use_scratch) {
    if (int rc = check_ptrs(work, {ws_d})) return rc;
  }
  if (!work) return BS_OK;
  if (int rc = check_grid(L, Z)) return rc;
  if (use_scratch) {
    if (int rc = bsa::bwd_scratch(&ws_d)) return rc;
  }
  log_call(use_scratch ? "attention_bwd_noalloc" : "attention_bwd", L, Z, d);
  bsa::BwdArgs a{Q, K, V, O, lse, dO, dQ, dK, dV, ws_d, Z, d, scale, causal, dt};
  a.am = attn_mask;
  a.kp = kp_mask;
  return bsa::launch_attention_bwd(L, a, (hipStream_t)stream);
}

extern "C" {

int bs_attention_bwd(bs_layout_t L, const void* Q, const void* K, const void* V, const void* O, const float* lse,
                     const void* dO, void* dQ, void* dK, void* dV, float* ws_d, int Z, int d, float scale, int flags,
                     const float* attn_mask, const float* kp_mask, bs_dtype dt, void* stream) {
  return attention_bwd(L, Q, K, V, O, lse, dO, dQ, dK, dV, ws_d, false, Z, d, scale, flags, attn_mask, kp_mask, dt,
                       stream);
}

int bs_attention_bwd_noalloc(bs_layout_t L, const void* Q, const void* K, const void* V, const void* O,
                             const float* lse, const void* dO, void* dQ, void* dK, void* dV, int Z, int d,
                             float scale, int flags, const float* attn_mask, const float* kp_mask, bs_dtype dt,
                             void* stream) {
  return attention_bwd(L, Q, K, V, O, lse, dO, dQ, dK, dV, nullptr, true, Z, d, scale, flags, attn_mask, kp_mask,
                       dt, stream);
}

int bs_dds(bs_layout_t L, const void* A, const float* S, void* C, int Z, int M, bs_dtype dt, void* stream) {
  return bs_dds_ex(L, A, S, C, Z, M, 0, dt, stream);
}

int bs_dds_ex(bs_layout_t L, const void* A, const float* S, void* C, int Z, int M, int trans, bs_dtype dt,
              void* stream) {
  if (int rc = check_handle(L)) return rc;
  if (trans & ~(BS_TRANS_A | BS_TRANS_B)) return fail(BS_ERR_INVALID_ARG, "unknown transpose flag");
  if (int rc = check_dtype(dt)) return rc;
  if (Z < 0 || M <= 0) return fail(BS_ERR_INVALID_ARG, "Z must be >= 0 and M > 0");
  if (M % 16) return fail(BS_ERR_UNSUPPORTED, "M must be a multiple of 16");
  const bool work = Z > 0;
  if (int rc = check_ptrs(work, {A, C})) return rc;
  if (work && L->nnz > 0) {
    if (int rc = check_ptrs(true, {S})) return rc;
  }
  if (!work) return BS_OK;
  if (int rc = check_grid(L, Z)) return rc;
  log_call("dds", L, Z, M);
  return bsa::launch_dds_ex(L, A, S, C, Z, M, trans, dt, (hipStream_t)stream);
}

int bs_attention(bs_layout_t L, const void* Q, const void* K, const void* V, void* O, int Z, int d, float scale,
                 int flags, bs_dtype dt, void* stream) {
  return bs_attention_fwd(L, Q, K, V, O, nullptr, Z, d, scale, flags, nullptr, nullptr, dt, stream);
}

int bs_attention_masked(bs_layout_t L, const void* Q, const void* K, const void* V, void* O, int Z, int d,
                        float scale, int flags, const float* attn_mask, const float* kp_mask, bs_dtype dt,
                        void* stream) {
  return bs_attention_fwd(L, Q, K, V, O, nullptr, Z, d, scale, flags, attn_mask, kp_mask, dt, stream);
}

int bs_attention_fwd(bs_layout_t L, const void* Q, const void* K, const void* V, void* O, float* lse, int Z, int d,
                     float scale, int flags, const float* attn_mask, const float* kp_mask, bs_dtype dt,
                     void* stream) {
  if (int rc = check_handle(L)) return rc;
  if (int rc = check_masks(attn_mask, kp_mask)) return rc;
  if (int rc = check_dtype(dt, true)) return rc;
  if (flags & ~BS_CAUSAL) return fail(BS_ERR_INVALID_ARG, "unknown flag");
  if (Z < 0) return fail(BS_ERR_INVALID_ARG, "Z must be >= 0");
  if (d != 64 && d != 128) return fail(BS_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (dt == BS_F8E4M3 && (d != 128 || L->block < 32))
    return fail(BS_ERR_UNSUPPORTED, "BS_F8E4M3 attention needs d = 128 and blocks of 32, 64 or 128");
  const bool causal = flags & BS_CAUSAL;
  if (causal && L->nbr != L->nbc) return fail(BS_ERR_INVALID_ARG, "causal attention needs a square layout");
  const bool work = Z > 0;
  if (int rc = check_ptrs(work, {Q, K, V, O})) return rc;
  if (!work) return BS_OK;
  if (int rc = check_grid(L, Z)) return rc;
  log_call("attention", L, Z, d);
  bsa::AttnArgs a{Q, K, V, O, Z, d, scale, causal, dt};
  a.am = attn_mask;
  a.kp = kp_mask;
  a.lse = lse;
  return bsa::launch_attention(L, a, (hipStream_t)stream);
}

}  // extern "C"
