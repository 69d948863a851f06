/*
 * i4s.h -- C ABI of libi4s: packed INT4 SparseGEMV over the 2-bit CSR format,
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed follows "Efficient LLM-based Advertising via Model
 * Compression and Parallel Verification" (arXiv 2605.11582):
 *   - section 3.2, "Sparsification", Eq. (3): N:M pruning by element
 *     importance |W_ij| * ||X_j||_2 + |W_ij| * |dE/dW_ij|; each aligned
 *     group of 4 columns keeps its n_keep most important weights (2 for 2:4,
 *     1 for 1:4, 4 = dense).  i4s_pack takes a constant activation norm and
 *     no gradient term, so the importance is |W_ij|; i4s_pack_ex takes the
 *     norms and gradients from the caller;
 *   - section 3.1 and 3.2, "Adaptive Group-Wise Quantization": symmetric INT4
 *     weight-only quantization with a group size chosen per layer;
 *   - section 3.3, "Sparse Index Structure": CSR rows whose column index is a
 *     2-bit position inside the group of 4, eight indices per uint16 word,
 *     filled from the least significant bits;
 *   - section 3.3, "Computational Acceleration" and section 1 (the SparseGemv
 *     kernel): y = W x with INT4 weights widened to fp16 in registers and the
 *     activations staged in on-chip shared memory (LDS on this GPU).
 *
 * FORMAT (version 1).  W is R x K (rows = output features), K % 64 == 0.
 *   nnz_row = K * n_keep / 4; nnz = R * nnz_row.  Element e of a row lies in
 *   4-column group t = e / n_keep and column 4*t + code_e; the kept columns of
 *   a group are listed in ascending order.
 *   row_ptr : int32[R+1], row_ptr[i] = i * nnz_row (in elements).
 *   vals    : uint8[nnz/2].  Row i starts at byte row_ptr[i]/2.  Each
 *             little-endian 32-bit word holds 8 consecutive elements
 *             e0..e7; nibble slot k (bits 4k..4k+3) holds element
 *             (0,2,4,6,1,3,5,7)[k].  Nibble u = q + 8, q in [-8, 7].
 *   codes   : uint16[nnz/8] (absent when n_keep == 4).  Element e's code is
 *             at bits 2*(e % 8) of word e / 8 of the row (row i starts at
 *             word row_ptr[i]/8).  For 2:4, bits 4p..4p+3 of a word are
 *             group p's pair (first | second << 2).
 *   scales  : fp16 bits [R][K/G], s = round_to_nearest_even_fp16(amax / 7)
 *             over the kept elements whose column lies in [gG, (g+1)G); an
 *             all-zero group has s = +0 and q = 0.
 *   q       : clamp(round_half_even(w / s), -8, 7), computed with a correctly
 *             rounded division.
 *   W_hat[i][4t + code_e] = s[i][(4t)/G] * q_e; all other entries are 0.
 *   Adaptive group size (group_size == 0): each G in {64, 128, 256} is tried
 *   and the one with the smallest exact sum over kept elements of
 *   (w - s*q)^2 wins, ties going to the larger G.
 *
 * CONVENTIONS.  Every pointer to tensor data is a DEVICE pointer unless
 * marked "host".  The caller owns all memory: the library never allocates or
 * frees device memory (i4s_run_noalloc uses a fixed array in the library's
 * code object instead of a caller workspace).  `stream` is a hipStream_t passed as void* (NULL is
 * the null stream).  All argument checks run before anything is enqueued; a
 * failed check returns I4S_ERR_INVALID_ARGUMENT (or another status) and
 * leaves every buffer untouched.  Errors raised by the HIP runtime come back
 * as I4S_ERR_DEVICE; the message of the last failing call on the calling
 * thread is available from i4s_last_error().  Faults inside a kernel surface
 * at the caller's next synchronisation.  No call aborts or throws.
 */
#ifndef I4S_H
#define I4S_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define I4S_FORMAT_VERSION 1
#define I4S_MAX_BATCH 16
#define I4S_MAX_MULTI 8
#define I4S_NOALLOC_SCRATCH_BYTES (32u << 20) /* static scratch of i4s_run_noalloc, per GPU */

typedef enum i4s_status {
  I4S_OK = 0,
  I4S_ERR_INVALID_ARGUMENT = 1,  /* a shape, pattern, pointer or size is invalid      */
  I4S_ERR_UNSUPPORTED = 2,       /* the current device is not gfx950                  */
  I4S_ERR_NONFINITE_WEIGHT = 3,  /* W holds an Inf or NaN                             */
  I4S_ERR_WORKSPACE_TOO_SMALL = 4,
  I4S_ERR_DEVICE = 5             /* a HIP runtime call failed                         */
} i4s_status;

/* A packed layer.  Plain data: every buffer is owned by the caller, the
 * struct can be copied freely and holds no hidden state. */
typedef struct i4s_packed {
  int32_t rows;        /* R                                                   */
  int32_t cols;        /* K, a multiple of 64                                 */
  int32_t n_keep;      /* 1, 2 or 4 kept per group of 4 (4 = dense INT4)      */
  int32_t group_size;  /* G in use: 64, 128 or 256                            */
  int64_t nnz;         /* R * K * n_keep / 4                                  */
  int32_t *row_ptr;    /* [R+1]                                               */
  uint8_t *vals;       /* [nnz/2]                                             */
  uint16_t *codes;     /* [nnz/8]; NULL when n_keep == 4                      */
  uint16_t *scales;    /* [R*K/G] fp16 bits                                   */
} i4s_packed;

/* Buffer sizes in bytes. */
typedef struct i4s_sizes {
  uint64_t row_ptr;
  uint64_t vals;
  uint64_t codes;      /* 0 when n_keep == 4                                  */
  uint64_t scales;     /* for adaptive G, sized for the smallest candidate (64) */
  uint64_t workspace;  /* scratch i4s_pack needs                              */
} i4s_sizes;

/* What i4s_pack decided.  SSE values are exact integers in units of 2^-48,
 * split into high and low 64-bit halves. */
typedef struct i4s_pack_report {
  int32_t group_size;      /* G chosen (or the fixed G)                       */
  int32_t n_candidates;    /* 3 when chosen adaptively, else 0                */
  int32_t candidates[3];   /* 64, 128, 256                                    */
  int32_t reserved;
  uint64_t sse_hi[3];
  uint64_t sse_lo[3];
} i4s_pack_report;

/* Sizes of the packed buffers and of the pack workspace for an R x K weight.
 * Host-only and pure: touches no device.  group_size 0 means adaptive.
 * Errors: I4S_ERR_INVALID_ARGUMENT for rows < 1, cols not a positive multiple
 * of 64 (or of every G in use), n_keep not in {1,2,4}, G not in
 * {0,64,128,256}, nnz >= 2^31, or out == NULL. */
i4s_status i4s_pack_sizes(int32_t rows, int32_t cols, int32_t n_keep,
                          int32_t group_size, i4s_sizes *out /* host */);

/* Prune, quantize and encode a dense fp16 weight (section 3.2 and 3.3 of the
 * page; see FORMAT above).
 *   w_fp16     : [rows][cols] fp16 bits, row-major, 16-byte aligned.
 *   group_size : 64, 128, 256, or 0 to choose per matrix by minimum SSE.
 *   workspace  : device scratch of at least i4s_pack_sizes().workspace bytes,
 *                16-byte aligned; its contents on entry do not matter.
 *   inout      : host struct whose row_ptr, vals, codes (unless n_keep == 4)
 *                and scales point at caller-owned device buffers of the sizes
 *                i4s_pack_sizes() reports, each 16-byte aligned.  On success
 *                rows, cols, n_keep, group_size and nnz are filled in.
 *   report     : optional host struct receiving the chosen G and the SSEs.
 * Enqueues its kernels on `stream` and synchronises that stream once to read
 * back the non-finite flag and, when adaptive, the SSE totals.
 * The output buffers, the workspace (its first i4s_pack_sizes().workspace
 * bytes) and w_fp16 must not overlap one another.
 * Errors: I4S_ERR_INVALID_ARGUMENT (checks as in i4s_pack_sizes, null or
 * misaligned pointers, overlapping buffers), I4S_ERR_WORKSPACE_TOO_SMALL,
 * I4S_ERR_NONFINITE_WEIGHT (the output buffers are then unspecified),
 * I4S_ERR_UNSUPPORTED (device is not gfx950), I4S_ERR_DEVICE. */
i4s_status i4s_pack(const uint16_t *w_fp16, int32_t rows, int32_t cols,
                    int32_t n_keep, int32_t group_size, void *workspace,
                    uint64_t workspace_bytes, i4s_packed *inout /* host */,
                    i4s_pack_report *report /* host, may be NULL */,
                    void *stream);

/* i4s_pack with the full importance score of Eq. (3) of the page (section
 * 3.2): |W_ij| * ||X_j||_2 + |W_ij| * |dE/dW_ij|.  The N:4 mask keeps the
 * n_keep elements of each aligned group of four columns with the largest
 * score, evaluated as |W_ij| * (n_j + |g_ij|) in fp32 with the sum and the
 * product each rounded to nearest even; among equal scores the lower column
 * is kept.  Same arguments and behaviour as i4s_pack plus:
 *   col_norm  : device, [cols] fp32 activation norms ||X_j||_2, 16-byte
 *               aligned, or NULL for n_j = 1.  Finite and >= 0 (-0 allowed).
 *   grad_fp16 : device, [rows][cols] fp16 bits of dE/dW, row-major, 16-byte
 *               aligned, or NULL for g_ij = 0.  Finite.
 * Both NULL gives exactly i4s_pack's magnitude mask, and so do norms that are
 * all 1 without gradients.  Only the mask depends on them: the kept weights
 * are quantized and encoded as in i4s_pack.  A score beyond fp32's range is
 * +inf and ties other +inf scores.  Both inputs are only read, and neither
 * may overlap an output buffer or the workspace.
 * Errors: as i4s_pack, plus I4S_ERR_INVALID_ARGUMENT for a misaligned
 * col_norm or grad_fp16, a negative or non-finite norm or a non-finite
 * gradient (detected on the device; a non-finite weight is reported first). */
i4s_status i4s_pack_ex(const uint16_t *w_fp16, int32_t rows, int32_t cols,
                       int32_t n_keep, int32_t group_size,
                       const float *col_norm /* device, may be NULL */,
                       const uint16_t *grad_fp16 /* device, may be NULL */,
                       void *workspace, uint64_t workspace_bytes,
                       i4s_packed *inout /* host */,
                       i4s_pack_report *report /* host, may be NULL */,
                       void *stream);

/* y = W_hat x for `batch` activation vectors (section 3.3 of the page: the
 * SparseGemv kernel over the 2-bit CSR format).
 *   w      : host descriptor filled by i4s_pack (or an equivalent layout);
 *            group_size must be 64, 128 or 256; vals 16-byte, codes 8-byte,
 *            row_ptr 4-byte and scales 2-byte aligned.  row_ptr is read:
 *            row i's elements start at row_ptr[i], which must lie in
 *            [0, nnz - nnz_row] and be a multiple of 16 * n_keep (one
 *            64-column unit); i4s_pack writes i * nnz_row.  An entry off
 *            that grid is moved onto it (clamped to the range, rounded down
 *            to a unit) before any weight is read at it, so such a
 *            descriptor gives unspecified outputs but no read outside the
 *            buffers.
 *   x_fp16 : [batch][cols] fp16 bits, contiguous, 16-byte aligned.
 *   batch  : 1 .. I4S_MAX_BATCH.
 *   y_fp16 : [batch][rows] fp16 bits, contiguous, 2-byte aligned; fully
 *            overwritten.  Must not overlap x or any packed buffer.
 * Accumulates in fp32 and rounds y to fp16 (nearest even).  One kernel
 * launch on `stream`; asynchronous; allocates nothing; never synchronises.
 * Errors: I4S_ERR_INVALID_ARGUMENT (descriptor inconsistent, null or
 * misaligned pointers, batch out of range, x/y overlap),
 * I4S_ERR_UNSUPPORTED, I4S_ERR_DEVICE. */
i4s_status i4s_run(const i4s_packed *w /* host */, const uint16_t *x_fp16,
                   int32_t batch, uint16_t *y_fp16, void *stream);

/* Bytes of device workspace i4s_run_ws needs for this layer and batch; 0
 * when the call needs none.  Only the 2:4 batch GEMV splits K across blocks,
 * and only where that is faster than the one-launch kernel over whole rows:
 * K > 32768 (beyond the one-launch kernel) at any batch >= 2; batch 3-8 with
 * K >= 8192 where the one-launch kernel would run fewer than 192 blocks
 * (fewer than 3072 rows, or 4800 to 6143 rows, where it takes two 16-row
 * tiles per block), and at batch 8 up to 256 blocks (4096 rows); batch 9-16
 * with K >= 5120 on at most 8192 rows; and not when K <= 1024 (a single
 * slice).  Host-only and pure.  Errors:
 * I4S_ERR_INVALID_ARGUMENT (descriptor inconsistent, batch out of range,
 * bytes == NULL). */
i4s_status i4s_run_workspace_size(const i4s_packed *w /* host */, int32_t batch,
                                  uint64_t *bytes /* host */);

/* y = W_hat x as i4s_run, using a caller workspace that lets the 2:4 batch
 * kernel split K across blocks (section 3.3 of the page: the activations of
 * a block's 1024-column slice are staged on chip once for up to 128 rows).
 * Same arguments as i4s_run plus:
 *   workspace       : device buffer of at least i4s_run_workspace_size()
 *                     bytes, 16-byte aligned (may be NULL when that size is
 *                     0).  Scratch for the fp32 partial sums of each slice:
 *                     its contents on entry do not matter and on return are
 *                     unspecified.  Calls that share a workspace must not
 *                     overlap (order them on one stream).  Must not overlap
 *                     x or y.
 *   workspace_bytes : its size.
 * Two kernel launches on `stream` when the workspace size is nonzero (the
 * sliced product, then the sum of the slices), one otherwise; asynchronous;
 * allocates nothing.  The result is deterministic: slices are added in a
 * fixed order.
 * Errors: as i4s_run, plus I4S_ERR_WORKSPACE_TOO_SMALL. */
i4s_status i4s_run_ws(const i4s_packed *w /* host */, const uint16_t *x_fp16,
                      int32_t batch, uint16_t *y_fp16, void *workspace,
                      uint64_t workspace_bytes, void *stream);

/* y_m = W_hat_m x for n layers that read the same activations (the q, k, v
 * projections of an attention block; the gate and up projections of an MLP),
 * in one kernel launch where possible: horizontal fusion, which pays the
 * per-launch cost once instead of n times (the SparseGemv of section 3.3 of
 * the page, applied to several weights at once).
 *   w      : host array of n descriptors as for i4s_run; every layer has the
 *            same cols.
 *   n      : 1 .. I4S_MAX_MULTI.
 *   x_fp16 : [batch][cols] fp16 bits, as for i4s_run, shared by all layers.
 *   y_fp16 : host array of n device pointers; y_fp16[m] is [batch][rows_m]
 *            fp16 bits, 2-byte aligned, fully overwritten.  The outputs must
 *            not overlap one another, x, or any layer's packed buffers.
 * Results are bit-identical to n i4s_run calls.  One launch when the layers
 * share n_keep and group_size and either batch is 1 and cols <= 16384, or
 * batch >= 2 and cols <= 32768 (except batch 2 with cols <= 4096 and a layer
 * of at most 8192 rows, which single calls run on another kernel, and layers
 * whose single calls split the row into chunks of different widths);
 * otherwise one launch per layer, in order, on `stream`.  Asynchronous; allocates nothing.
 * Errors: as i4s_run (reported for the first offending layer), plus
 * I4S_ERR_INVALID_ARGUMENT for n out of range, NULL arrays, differing cols
 * or overlapping outputs. */
i4s_status i4s_run_multi(const i4s_packed *w /* host, n entries */, int32_t n,
                         const uint16_t *x_fp16, int32_t batch,
                         uint16_t *const *y_fp16 /* host, n device pointers */,
                         void *stream);

/* i4s_run_ws for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * workspace is a static array inside the library, I4S_NOALLOC_SCRATCH_BYTES
 * per GPU, held from the first call on that GPU until the process ends.
 * Same arguments, kernels and results (bit for bit) as i4s_run_ws with a
 * caller workspace; calls no allocating routine.
 * Every call on a GPU shares that GPU's array and leaves its contents
 * behind (nothing in it needs clearing: the partial sums are written before
 * they are read in the same call), so calls that may overlap on one GPU --
 * on different streams, or from several threads without ordering -- race
 * and must not be made.
 * Errors: as i4s_run, plus I4S_ERR_WORKSPACE_TOO_SMALL when
 * i4s_run_workspace_size() exceeds I4S_NOALLOC_SCRATCH_BYTES (checked before
 * anything is enqueued; such a layer needs i4s_run_ws). */
i4s_status i4s_run_noalloc(const i4s_packed *w /* host */, const uint16_t *x_fp16,
                           int32_t batch, uint16_t *y_fp16, void *stream);

/* Static text for a status code (never NULL). */
const char *i4s_status_string(i4s_status s);

/* Message of the last failing call on the calling thread ("" if none). */
const char *i4s_last_error(void);

/* Library version: 10000 * major + 100 * minor + patch. */
int32_t i4s_version(void);

/* FORMAT version this library reads and writes (I4S_FORMAT_VERSION). */
int32_t i4s_format_version(void);

#ifdef __cplusplus
}
#endif

#endif /* I4S_H */
