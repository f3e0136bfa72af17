/*
 * bsattn.h -- block-sparse multi-head attention for AMD MI355X (gfx950).
 *
 * The operations are the ones the Triton issue "question on blocksparse"
 * (openai/triton #117) names for block-sparse matrix products:
 *   SDD  sparse = dense x dense   (sampled dense-dense product)
 *   DSD  dense  = sparse x dense  (left operand sparse)
 *   DDS  dense  = dense x sparse  (right operand sparse)
 * plus the block-sparse row softmax that runs on the SDD output, and the
 * attention those three compose (SDD -> softmax -> DSD), here fused into one
 * kernel. The sparsity layout is a tensor of 0s and 1s, one entry per
 * non-overlapping square block of 16, 32, 64 or 128 (same answer). Regular
 * layouts may instead be given in the affine-compressed row form (ACSR) of
 * the SPLAT abstract (NSF-PAR, Jain).
 *
 * Conventions for every call
 *  - Tensor pointers are DEVICE pointers to contiguous row-major memory on
 *    the current HIP device, unless a parameter says "host".
 *  - The caller owns and pre-allocates every tensor. The library allocates
 *    device memory only inside bs_layout_build*, and frees it in
 *    bs_layout_free.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Compute calls are asynchronous on it; pointers must stay valid until
 *    the work completes. bs_layout_build*, bs_layout_export synchronise
 *    the stream.
 *  - Every call returns BS_OK (0) or a negative bs_status. Arguments are
 *    validated before any HIP call is made; bs_last_error() gives the
 *    message of the last failure on the calling thread.
 *  - A layout handle's tables are immutable after it is built, and the
 *    handle may be used from several streams and threads at once; its one
 *    setting, bs_layout_set_kv_share, is read when a call is issued.
 *
 * Shapes (b = block, nnz = number of stored blocks over all heads)
 *  - layout                 uint8 [H][nbr][nbc], values 0 or 1, one layout
 *                           per head, shared across the batch Z.
 *  - block ids              stored blocks enumerated in (head, block-row,
 *                           block-col) lexicographic order; the k-th gets k.
 *  - block-sparse tensor    float32 [Z][nnz][b][b]; block k row-major.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct bs_layout* bs_layout_t;

/* element type of the dense operands (block-sparse tensors are always
   float32): IEEE binary32, bfloat16 or IEEE binary16. With the 16-bit types
   the products run on the 16-bit matrix cores with float32 accumulation;
   float32 values that feed a product (P, S) are rounded to the operand type
   (round to nearest even) and results are rounded once at the end.
   BS_F8E4M3 (fused attention only: bs_attention, bs_attention_masked,
   bs_attention_fwd; d = 128 and blocks of 32, 64 or 128): Q and K are OCP
   FP8 E4M3 bytes, taken as the values they encode (no scale factors), and
   the score product runs on the fp8 matrix cores (exact products, float32
   accumulation); V and O are bfloat16 and P is rounded to bfloat16 for the
   P.V product, as with BS_BF16. Every other call returns
   BS_ERR_UNSUPPORTED for it. */
typedef enum { BS_F32 = 0, BS_BF16 = 1, BS_F16 = 2, BS_F8E4M3 = 3 } bs_dtype;

/* flags for bs_softmax / bs_attention */
enum { BS_CAUSAL = 1 };

/* operand flags for bs_sdd_ex / bs_dsd_ex / bs_dds_ex */
enum { BS_TRANS_A = 1, BS_TRANS_B = 2 };

typedef enum {
  BS_OK = 0,
  BS_ERR_INVALID_ARG = -1, /* null pointer with work to do, negative size,
                              causal on a non-square layout, unknown flag */
  BS_ERR_UNSUPPORTED = -2, /* block not in {16,32,64,128}; head_dim not in
                              {64,128}; a dimension not a multiple of 16 */
  BS_ERR_LAYOUT = -3,      /* a layout value other than 0 or 1 */
  BS_ERR_SHAPE = -4,       /* sizes overflow the 32/64-bit index ranges */
  BS_ERR_HIP = -5,         /* a HIP runtime call failed */
  BS_ERR_OOM = -6,         /* device allocation failed (also forced, with
                              no allocation attempted, when the environment
                              variable BS_FAULT_INJECT is "oom") */
  BS_ERR_NO_DEVICE = -7    /* no HIP device is visible */
} bs_status;

/* One affine row term of an ACSR layout: every block row r in
   [row_begin, row_end) stores the block columns
   slope*r + offset + stride*k, k = 0 .. count-1, that fall in [0, nbc).
   A layout is the union of its terms (SPLAT abstract: affine-compressed
   sparse rows for the regular geometry of sparse-MHSA patterns). */
typedef struct {
  int32_t row_begin, row_end, slope, offset, stride, count;
} bs_acsr_term;

/* Build a layout handle from a 0/1 layout.
   layout: DEVICE uint8 [H][nbr][nbc]. block in {16,32,64,128}.
   On success *out owns device tables: block-CSR (row_ptr, col_idx) over
   (h, r, c) and CSC (col_ptr, row_idx, blk_id) over (h, c, r), built on the
   GPU. Errors: BS_ERR_UNSUPPORTED (block), BS_ERR_LAYOUT (a value not 0/1),
   BS_ERR_INVALID_ARG, BS_ERR_SHAPE, BS_ERR_OOM, BS_ERR_HIP. Synchronises
   `stream`. *out is NULL on failure. */
int bs_layout_build(const uint8_t* layout, int H, int nbr, int nbc, int block,
                    void* stream, bs_layout_t* out);

/* Build a layout handle from ACSR terms (HOST array of n_terms entries),
   the same pattern for every head. The terms are expanded on the GPU, then
   the same tables as bs_layout_build are built. Errors as bs_layout_build;
   a term with row_begin > row_end or count < 0 is BS_ERR_INVALID_ARG. */
int bs_layout_build_acsr(const bs_acsr_term* terms, int n_terms, int H,
                         int nbr, int nbc, int block, void* stream,
                         bs_layout_t* out);

/* Number of stored blocks of a handle, summed over heads (the length of
   the block-sparse tensors' nnz axis). nnz: host int64_t. Errors:
   BS_ERR_INVALID_ARG for a NULL handle or output pointer. */
int bs_layout_nnz(bs_layout_t L, int64_t* nnz);

/* K/V sharing across block rows (SPLAT abstract: the regular geometry of
   an ACSR pattern, analysed when the handle is built). On a handle from
   bs_layout_build_acsr whose terms all have slope 1 and cover every row,
   row r holds the columns r + o for o in one offset set, so rows r and
   r + t share the columns that the set and its shift by t have in common.
   The handle keeps a plan when two rows r and r + stride hold at least 1.5
   times as many blocks as the union of their columns, for the stride (1 to
   64) with the smallest union (blocks of 32 or more). When the plan is used
   (bs_layout_set_kv_share), the fused attention without dense masks runs
   `rows` = 2 block rows r0, r0 + stride per workgroup and stages each K/V
   block of their union once: float32 with blocks of 32 (head_dim 64 or
   128) or 64 (head_dim 64), and bf16 / fp16 with blocks of 32 to 128. Each
   row still adds up its own blocks in ascending column order with the same
   arithmetic as the one-row kernel, so the output has the same bits as
   without sharing whenever the one-row kernel runs one key group per row.
   bs_layout_kv_share reports the plan: *rows = 1 and *stride = 0 when the
   handle has none. Errors: BS_ERR_INVALID_ARG for a NULL handle or output
   pointer. */
int bs_layout_kv_share(bs_layout_t L, int* rows, int* stride);

/* Use of the sharing plan by the fused attention: mode 1 wherever it
   applies, 0 never (one block row per workgroup), -1 (the default) where
   it measured faster: bf16 / fp16 with blocks of 64 (strided band, 16384
   tokens: 3% at head_dim 128, 6-7% at 64). Float32 measured the same time
   either way (389 and 391 us on strided_acsr_b32, a kernel bound by the
   matrix cores rather than by staging); bf16 with blocks of 128 measured
   12-16% slower with it. Read when a call is issued (calls already on a
   stream keep their kernel); not synchronised with calls on the same handle
   from other host threads. Errors: BS_ERR_INVALID_ARG for a NULL handle or
   a mode other than -1, 0 or 1. */
int bs_layout_set_kv_share(bs_layout_t L, int mode);

/* Sizes of a handle (any output pointer may be NULL). */
int bs_layout_info(bs_layout_t L, int* H, int* nbr, int* nbc, int* block,
                   int64_t* nnz);

/* Copy the tables to HOST buffers (any may be NULL): row_ptr[H*nbr+1],
   col_idx[nnz], col_ptr[H*nbc+1], row_idx[nnz], blk_id[nnz]. Synchronous. */
int bs_layout_export(bs_layout_t L, int32_t* row_ptr, int32_t* col_idx,
                     int32_t* col_ptr, int32_t* row_idx, int32_t* blk_id);

/* Release a handle (NULL is ignored). Call it when no queued work still
   uses the handle. */
void bs_layout_free(bs_layout_t L);

/* SDD: S[z,k] = A[z,h,r-block,:] . B[z,h,c-block,:]^T for every stored block
   k = (h, r, c); the sampled dense-dense product of the issue's first mode,
   in attention S = Q K^T.
   A: [Z][H][nbr*b][K], B: [Z][H][nbc*b][K] of dtype dt; S: float32
   [Z][nnz][b][b]. K > 0 and a multiple of 16. */
int bs_sdd(bs_layout_t L, const void* A, const void* B, float* S, int Z,
           int K, bs_dtype dt, void* stream);

/* Block-sparse row softmax (the issue's softmax on SDD output; the same as
   full-attention softmax over the stored entries). For query row i of
   block row r of head h, x = scale * S over every stored block (h, r, c);
   with BS_CAUSAL, entries whose key index c*b+j exceeds the query index
   r*b+i are -inf (the dense mask inside diagonal blocks). P = exp(x - max) /
   sum exp(x - max); a row with no visible entry is all zeros.
   S, P: float32 [Z][nnz][b][b]; P may equal S (in place). BS_CAUSAL needs
   nbr == nbc. */
int bs_softmax(bs_layout_t L, const float* S, float* P, int Z, float scale,
               int flags, void* stream);

/* ---- dense masks (question on blocksparse: dense masks may be passed
   alongside the layout; the format is not given there, the one below is
   this library's) ----
   attn_mask: float32 [nbr*b][nbc*b], indexed by global query and key,
     shared by every batch element and head; may be NULL.
   kp_mask (key padding): float32 [Z][nbc*b], per batch element and key;
     may be NULL.
   Both are added to scale*S before the causal mask and the row softmax;
   -inf hides an entry, a row with every entry hidden gives zeros. Entries
   outside the layout's blocks stay hidden whatever the masks hold. +inf or
   NaN in a mask gives NaN outputs. Both pointers must be 16-byte aligned
   (BS_ERR_INVALID_ARG otherwise); the caller keeps ownership. With both
   NULL each masked call is its unmasked counterpart. */

/* bs_softmax with the dense masks above. */
int bs_softmax_masked(bs_layout_t L, const float* S, float* P, int Z,
                      float scale, int flags, const float* attn_mask,
                      const float* kp_mask, void* stream);

/* DSD: C[z,h,r-block,:] = sum over stored (h,r,c) of P[z,k] . B[z,h,c-block,:]
   (the issue's second mode; in attention O = P V).
   P: float32 [Z][nnz][b][b]; B: [Z][H][nbc*b][Nd], C: [Z][H][nbr*b][Nd] of
   dtype dt (16-bit types: P is rounded to dt for the product, C is rounded
   from the float32 accumulator). Rows with no stored block are written as
   zero.
   Nd > 0 and a multiple of 16. */
int bs_dsd(bs_layout_t L, const float* P, const void* B, void* C, int Z,
           int Nd, bs_dtype dt, void* stream);

/* DDS: C[z,h,:,c-block] = sum over stored (h,r,c) of A[z,h,:,r-block] . S[z,k]
   (the issue's third mode; in attention's backward dV^T = dO^T P).
   A: [Z][H][M][nbr*b], C: [Z][H][M][nbc*b] of dtype dt; S: float32
   [Z][nnz][b][b]. Columns with no stored block are written as zero.
   M > 0 and a multiple of 16. */
int bs_dds(bs_layout_t L, const void* A, const float* S, void* C, int Z,
           int M, bs_dtype dt, void* stream);

/* Fused block-sparse attention: O = softmax(scale Q K^T + mask) V with the
   mask of the layout (and BS_CAUSAL), i.e. SDD -> softmax -> DSD in one
   kernel (the issue's attention composition) with a streaming row softmax
   (running max and sum, Triton tutorial Puzzles 8 and 9); P never leaves
   the chip. Q: [Z][H][nbr*b][d], K, V: [Z][H][nbc*b][d], O: [Z][H][nbr*b][d],
   all of dtype dt; d in {64, 128}. 16-bit types: scores and softmax in
   float32, P rounded to dt for the P.V product, O rounded from float32.
   Rows with no visible key are zero. */
int bs_attention(bs_layout_t L, const void* Q, const void* K, const void* V,
                 void* O, int Z, int d, float scale, int flags, bs_dtype dt,
                 void* stream);

/* bs_attention with the dense masks above (fused: the masks are read at the
   stored blocks only). */
int bs_attention_masked(bs_layout_t L, const void* Q, const void* K,
                        const void* V, void* O, int Z, int d, float scale,
                        int flags, const float* attn_mask,
                        const float* kp_mask, bs_dtype dt, void* stream);

/* The forward of the fused backward below: bs_attention_masked that also
   writes lse (may be NULL), float32 [Z][H][nbr*b]: for every query row the
   natural log of its softmax denominator, log sum_j exp(x_j) over the
   visible entries of x = scale*S + masks (-inf for a row with no visible
   key), so that P = exp(x - lse). Caller-owned. */
int bs_attention_fwd(bs_layout_t L, const void* Q, const void* K,
                     const void* V, void* O, float* lse, int Z, int d,
                     float scale, int flags, const float* attn_mask,
                     const float* kp_mask, bs_dtype dt, void* stream);

/* ---- backward (the exact gradient of the forward above) ----
   The attention gradient is made of the same three modes (the issue's
   SDD / DSD / DDS) plus the softmax gradient; the autograd pattern (forward
   kernel, backward kernel, one autograd function) is the Triton tutorial's.
   With P the softmax output and dO = dL/dO:
     dV = P^T dO, dP = dO V^T, dS = scale * P * (dP - rowsum(P * dP)),
     dQ = dS K, dK = dS^T Q. */

/* Gradient of bs_softmax with respect to S, given its output P and
   dP = dL/dP: for query row i of block row r of head h,
   D = sum over the row's stored entries of P * dP, and
   dS = scale * P * (dP - D); entries the mask hid (P = 0) get zero.
   P, dP, dS: float32 [Z][nnz][b][b]; dS may equal dP or P (in place). */
int bs_softmax_backward(bs_layout_t L, const float* P, const float* dP,
                        float* dS, int Z, float scale, void* stream);

/* DSD of the transposed block matrix:
   C[z,h,c-block,:] = sum over stored (h,r,c) of S[z,k]^T . B[z,h,r-block,:]
   (in attention's backward dK = dS^T Q and dV = P^T dO).
   S: float32 [Z][nnz][b][b]; B: [Z][H][nbr*b][Nd], C: [Z][H][nbc*b][Nd] of
   dtype dt (16-bit types: S is rounded to dt for the product, C is rounded
   from the float32 accumulator). Block columns with no stored block are written
   as zero. Nd in {64, 128}. */
int bs_dsd_t(bs_layout_t L, const float* S, const void* B, void* C, int Z,
             int Nd, bs_dtype dt, void* stream);

/* Backward of bs_attention: dQ, dK, dV from Q, K, V and dO, recomputing P
   (SDD, softmax), then dP = SDD(dO, V), dS = softmax gradient,
   dQ = DSD(dS, K), dK = DSD^T(dS, Q), dV = DSD^T(P, dO). Shapes and dtype
   as bs_attention (dQ like Q, dK and dV like K); d in {64, 128}.
   ws_s and ws_p are caller-owned float32 workspaces of Z*nnz*b*b elements
   each (the library allocates nothing here); on return ws_p holds P. */
int bs_attention_backward(bs_layout_t L, const void* Q, const void* K,
                          const void* V, const void* dO, void* dQ, void* dK,
                          void* dV, float* ws_s, float* ws_p, int Z, int d,
                          float scale, int flags, bs_dtype dt, void* stream);

/* Backward of bs_attention_masked: as bs_attention_backward, with P
   recomputed under the same dense masks (the masks are constants: they get
   no gradient). */
int bs_attention_backward_masked(bs_layout_t L, const void* Q, const void* K,
                                 const void* V, const void* dO, void* dQ,
                                 void* dK, void* dV, float* ws_s, float* ws_p,
                                 int Z, int d, float scale, int flags,
                                 const float* attn_mask, const float* kp_mask,
                                 bs_dtype dt, void* stream);

/* Fused backward: dQ, dK, dV of bs_attention_fwd from its inputs, its
   output O and lse, and dO = dL/dO, without materialising S or P: with
   x = scale*S + masks and D = rowsum(dO * O) (which equals rowsum(P * dP)),
   P = exp(x - lse), dS = scale * P * (dO V^T - D), dQ = dS K, dK = dS^T Q,
   dV = P^T dO (the same gradient as bs_attention_backward_masked). Two
   kernels: one over block rows (dQ, and the rows' D terms into ws_d), one
   over block columns (dK, dV). Q, O, dO, dQ: [Z][H][nbr*b][d]; K, V, dK, dV:
   [Z][H][nbc*b][d], all of dtype dt; d in {64, 128}. lse: float32
   [Z][H][nbr*b] as bs_attention_fwd wrote it, with the same scale, flags
   and masks. ws_d: caller-owned float32 workspace of Z*H*nbr*b elements
   (its contents afterwards are unspecified). 16-bit types: P and dS (or
   dS / scale, the scale then applied to dQ and dK) are rounded to dt for
   the products. */
int bs_attention_bwd(bs_layout_t L, const void* Q, const void* K,
                     const void* V, const void* O, const float* lse,
                     const void* dO, void* dQ, void* dK, void* dV,
                     float* ws_d, int Z, int d, float scale, int flags,
                     const float* attn_mask, const float* kp_mask,
                     bs_dtype dt, void* stream);

/* bs_attention_bwd for callers that cannot allocate device memory (code
   under HIP graph capture, tight serving loops, harnesses that forbid
   hipMalloc): the same kernels and results, with D kept in a library-owned
   static device array of 2^21 float32 (8 MiB per device, held until the
   process ends) instead of a caller workspace. Makes no allocation of any
   kind. Errors as bs_attention_bwd, plus BS_ERR_SHAPE when Z*H*nbr*b
   exceeds 2^21 query rows. Every call on one device shares that device's
   array, so calls that may overlap on one device (several streams or
   threads) race and must be serialised by the caller; nothing in the array
   needs to start at zero (each call writes D before it reads it). */
int bs_attention_bwd_noalloc(bs_layout_t L, const void* Q, const void* K,
                             const void* V, const void* O, const float* lse,
                             const void* dO, void* dQ, void* dK, void* dV,
                             int Z, int d, float scale, int flags,
                             const float* attn_mask, const float* kp_mask,
                             bs_dtype dt, void* stream);

/* ---- the three modes with transposed operands (question on blocksparse:
   the three modes; the flags follow the usual matmul convention of
   operands used transposed) ----
   bs_sdd_ex: S[z,k] = A'[z,h,r-block,:] . B'[z,h,c-block,:]^T with
     A' = A stored [Z][H][nbr*b][K], or, with BS_TRANS_A, stored as
     [Z][H][K][nbr*b] (A' is its transpose); B' likewise with BS_TRANS_B:
     [Z][H][nbc*b][K] or [Z][H][K][nbc*b]. trans = 0 is bs_sdd.
   bs_dsd_ex: C = S' B' over the block matrix S' = S (block rows walked) or,
     with BS_TRANS_A, its transpose (block columns walked, blocks
     transposed: bs_dsd_t). B' is [Z][H][nb_in*b][Nd], or with BS_TRANS_B
     stored as [Z][H][Nd][nb_in*b]; C: [Z][H][nb_out*b][Nd], where
     (nb_in, nb_out) = (nbc, nbr), or (nbr, nbc) with BS_TRANS_A.
   bs_dds_ex: C = A' S' with S' = S or, with BS_TRANS_B, its transpose;
     A' is [Z][H][M][nb_in*b], or with BS_TRANS_A stored as
     [Z][H][nb_in*b][M]; C: [Z][H][M][nb_out*b], where (nb_in, nb_out) =
     (nbr, nbc), or (nbc, nbr) with BS_TRANS_B.
   Dtypes, sizes (K, Nd, M multiples of 16), empty rows / columns and errors
   as the plain calls; other flag bits are BS_ERR_INVALID_ARG. Layouts the
   plain calls cover run on their kernels; the others on a general kernel
   that gathers the transposed operands. */
int bs_sdd_ex(bs_layout_t L, const void* A, const void* B, float* S, int Z,
              int K, int trans, bs_dtype dt, void* stream);
int bs_dsd_ex(bs_layout_t L, const float* S, const void* B, void* C, int Z,
              int Nd, int trans, bs_dtype dt, void* stream);
int bs_dds_ex(bs_layout_t L, const void* A, const float* S, void* C, int Z,
              int M, int trans, bs_dtype dt, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* bs_last_error(void);

/* Library ABI version (major*10000 + minor*100 + patch). */
int bs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
