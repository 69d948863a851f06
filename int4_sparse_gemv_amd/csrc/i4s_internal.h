// Internal declarations shared by the host layer and the kernel launchers of
// libi4s.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "i4s.h"

namespace i4s {

// Columns covered by one "segment": the unit of work of a pack thread and of
// a GEMV lane.  Every supported group size (64, 128, 256) is a multiple of it,
// so a segment never straddles two quantization groups.
constexpr int kSegCols = 64;

// Pack workspace layout (bytes from the workspace base):
//   [0, 4)     uint32 flag bits: 1 non-finite weight, 2 negative or
//              non-finite column norm, 4 non-finite gradient
//   [16, 64)   three 128-bit SSE totals (lo, hi) for G = 64, 128, 256
//   [64, ...)  per-block 128-bit partials, 3 per analyze block
constexpr size_t kWsFlagOffset = 0;
constexpr size_t kWsTotalsOffset = 16;
constexpr size_t kWsPartialsOffset = 64;
constexpr int kPackThreads = 256;

inline int64_t pack_threads_total(int32_t rows, int32_t cols) {
  return (int64_t)rows * (cols / kSegCols);
}
inline int64_t pack_blocks(int32_t rows, int32_t cols) {
  return (pack_threads_total(rows, cols) + kPackThreads - 1) / kPackThreads;
}
inline size_t pack_workspace_bytes(int32_t rows, int32_t cols) {
  return kWsPartialsOffset + (size_t)pack_blocks(rows, cols) * 3 * 16;
}

constexpr uint32_t kPackFlagNonfiniteWeight = 1u, kPackFlagBadNorm = 2u, kPackFlagBadGrad = 4u;

// Pack kernels (i4s_pack.hip).  `adaptive` selects whether the analyze pass
// also accumulates the exact SSE of every candidate group size; it always
// raises the flag bits.  col_norm ([cols] fp32) and grad ([rows][cols] fp16)
// are the optional importance inputs (null when absent).
hipError_t launch_pack_analyze(const uint16_t *w, const float *col_norm, const uint16_t *grad,
                               int32_t rows, int32_t cols, int32_t n_keep, bool adaptive, void *ws,
                               hipStream_t stream);
hipError_t launch_pack_emit(const uint16_t *w, const float *col_norm, const uint16_t *grad,
                            int32_t rows, int32_t cols, int32_t n_keep, int32_t group_size,
                            const i4s_packed &out, hipStream_t stream);

// Layers of one fused launch (i4s_run_multi): block b belongs to the first
// layer m with b < block_end[m]; its blocks are numbered from the previous
// layer's block_end.  Passed by value as a kernel argument.
constexpr int kMaxMulti = I4S_MAX_MULTI;
struct MultiDesc {
  int32_t n;
  int32_t block_end[kMaxMulti];
  int32_t rows[kMaxMulti];
  int32_t sg_shift[kMaxMulti];
  const int32_t *row_ptr[kMaxMulti];
  const uint8_t *vals[kMaxMulti];
  const uint16_t *codes[kMaxMulti];
  const uint16_t *scales[kMaxMulti];
  uint16_t *y[kMaxMulti];
};

// GEMV kernels.  launch_gemv (i4s_gemv_batch.hip) dispatches every call;
// launch_gemv_b1 (i4s_gemv_b1.hip) runs batch 1 for n_keep 2 and 4.
hipError_t launch_gemv_b1(const i4s_packed &w, const uint16_t *x, uint16_t *y, hipStream_t stream);
// Batch 2 on the VALU for layers of at most 8192 rows and K <= 4096 (each
// unit decoded once, then multiplied with both vectors); returns
// hipErrorNotSupported (launching nothing) where it does not apply.
hipError_t launch_gemv_bv(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                          hipStream_t stream);
bool gemv_bv_applies(const i4s_packed &w, int32_t batch);
// Fused batch-1 launch of n layers with one n_keep and K <= 16384; returns
// hipErrorNotSupported (launching nothing) when the layers do not fit it.
hipError_t launch_gemv_b1_multi(const i4s_packed *w, int32_t n, const uint16_t *x, uint16_t *const *y,
                                hipStream_t stream);
// Every layer of an i4s_run_multi call: one launch when a fused kernel
// covers them, else one launch per layer in order.
hipError_t launch_gemv_multi(const i4s_packed *w, int32_t n, const uint16_t *x, int32_t batch,
                             uint16_t *const *y, hipStream_t stream);
hipError_t launch_gemv(const i4s_packed &w, const uint16_t *x, int32_t batch,
                       uint16_t *y, hipStream_t stream);

// K split of the batch 2:4 GEMV across blocks (needs a caller workspace):
// ksplit slices of kKUnits 64-column units x row_groups groups of
// kKWaves * tw 16-row tiles.  The workspace holds the fp32 partial tiles of
// every slice (scratch: read only after being written in the same call).
// ksplit == 0 means "no split kernel" (batch 1, not 2:4, or a shape the rows
// kernel runs faster) and a workspace of 0 bytes; ksplit == 1 runs the split
// kernel without partials (0 bytes).
// Kernel-choice thresholds.  Fixed when the library is built (nothing read
// at run time changes which kernel runs); a build may override them with -D
// to measure the alternatives (python -m int4_sparse_gemv_amd.build --define).
//   I4S_BATCH2_VALU_MAX_ROWS / _MAX_K: batch 2 runs on the two-vector VALU
//     kernel for layers of at most this many rows and columns (0 rows: never);
//   I4S_MATRIX_CORE_MIN_BATCH: from this batch up, layers run on the matrix
//     cores (the VALU batch kernel below it, and for shapes the matrix-core
//     kernels do not cover).
#ifndef I4S_BATCH2_VALU_MAX_ROWS
#define I4S_BATCH2_VALU_MAX_ROWS 8192
#endif
#ifndef I4S_BATCH2_VALU_MAX_K
#define I4S_BATCH2_VALU_MAX_K 4096
#endif
#ifndef I4S_MATRIX_CORE_MIN_BATCH
#define I4S_MATRIX_CORE_MIN_BATCH 2
#endif
#ifndef I4S_SPLIT_TW2_MIN_BLOCKS
#define I4S_SPLIT_TW2_MIN_BLOCKS 384
#endif

// Shapes shared by the batch kernels (i4s_gemv_batch.hip) and the host-side
// plan of a call (i4s_plan.cpp).
constexpr int kKWaves = 4;                       // K-split kernel: waves per block
constexpr int kKUnits = 16;                      // K-split kernel: units per slice
// K-split kernel: halfs per staged vector, 16 halfs of padding: 520 dwords,
// 8 banks on per vector, so the B reads of 8 vectors x 2 column quarters in
// one LDS pass fall in distinct banks (8 halfs of padding put vector v + 1
// of quarter q on the banks of vector v of quarter q + 1: 24-36 % of the LDS
// cycles in conflict at batch 4-8)
constexpr int kKXStride = kKUnits * kSegCols + 16;
constexpr int kKPartialTileBytes = 64 * 16;      // one fp32 16x16 partial tile (64 lanes x 4 floats)
constexpr int kRUnits = 16;                      // rows kernel: units per chunk (the wide form)
constexpr int kRMaxWaves = 8;                    // rows kernel: waves per block (the wide form)

// Geometry of a chunk of U units (16 or 8) in a wave's LDS area for one
// tile: vals [16 rows][U + 1] (the extra column spreads the banks), codes
// [16 rows][U + 1], scales [U units][kScaleStride] (16 rows and 4 halfs of
// padding: the 64 lanes' 2-byte writes of one load, unit lu of rows
// 4k..4k+3, then fall in distinct banks -- with 16 halfs per unit units lu
// and lu + 8 shared banks, 28 % of the LDS cycles in conflict -- and the
// 8-byte reads of 4 rows stay aligned).  One load instruction covers 64 / U
// rows of U units (4 rows x 256 bytes or 8 rows x 128 bytes of vals).
template <int U, int NK = 2>
struct RowsGeom {
  static constexpr int kStride = U + 1;
  // vals per unit-row: 16 bytes (2:4), 8 (1:4: the 2:4 layout, half used), 32 (dense)
  static constexpr int kValsBytes = 16 * kStride * (NK == 4 ? 32 : 16);
  static constexpr int kCodesBytes = NK == 4 ? 0 : 16 * kStride * 8;
  static constexpr int kScaleStride = 20;
  static constexpr int kTileLds = kValsBytes + kCodesBytes + U * kScaleStride * 2;  // 2:4 and 1:4: 7168 / 3776 bytes
  static constexpr int kRowsPerLoad = 64 / U;
  static constexpr int kLoads = 16 / kRowsPerLoad;  // load instructions per tile and chunk
  static constexpr int kBlocks = U / 4;             // 4-unit blocks per chunk
  static constexpr int kMaxWaves = U == 8 ? 16 : 8;
};

// Rows kernel with compact B fragments: the activations of a 4-unit block
// pass through this much of the wave's LDS area (4 vectors x 4 units x 128
// bytes at once, 8 vectors x 2 units twice, or 16 vectors x 1 unit four
// times).
constexpr int kRowsBcBytes = 2048;

// Launch shape of the rows kernel for one layer: chunk width u (8 or 16
// units), chunks per wave cpw, waves per block, 16-row tiles per wave tpw,
// how the B fragments are read (bv = 4, 8 or 16: at most that many vectors,
// read once and spread through the wave's LDS area; bv = 0: each lane reads
// its own) and
// the block's dynamic LDS.  rows_shape only returns combinations that the
// batch kernels instantiate: u 16 with (cpw, tpw) in {(1, 1), (1, 2), (2, 1),
// (2, 2) but not dense, (4, 1)}; u 8 with cpw 1 and tpw in {1, 2, 4 for 2:4
// only}; bv 4 or 8 only with tpw 1 or 2 (for 1:4 only with u 8 and cpw 1),
// bv 16 only with tpw 1, or tpw 4 for 2:4.  units must satisfy the rows kernel's
// limit (K <= 32768).
struct RowsShape {
  int u = 0, cpw = 0, waves = 0, tpw = 0, bv = 0;
  size_t lds = 0;
};
RowsShape rows_shape(int units, int total_tiles, int batch, int n_keep, int want_u = 0);

struct SplitPlan {
  int row_groups = 0, ksplit = 0, tw = 0;
  size_t partial_bytes = 0, workspace_bytes = 0;
};
SplitPlan split_plan(const i4s_packed &w, int32_t batch);
hipError_t launch_gemv_ws(const i4s_packed &w, const uint16_t *x, int32_t batch,
                          uint16_t *y, const SplitPlan &plan, void *workspace,
                          hipStream_t stream);

// Device address of the current device's static scratch array
// (I4S_NOALLOC_SCRATCH_BYTES, i4s_noalloc.hip), looked up once per device.
hipError_t noalloc_scratch(void **ptr);

}  // namespace i4s
