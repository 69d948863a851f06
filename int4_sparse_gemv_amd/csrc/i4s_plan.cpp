// Host-side plan of a GEMV call: whether the 2:4 batch GEMV splits K across
// blocks, and the workspace that needs (i4s_run_workspace_size, i4s_run_ws,
// i4s_run_noalloc).  Plain host code: no device code, no HIP calls.

#include "i4s_internal.h"

namespace i4s {

SplitPlan split_plan(const i4s_packed &w, int32_t batch) {
  SplitPlan pl{};
  if (w.n_keep != 2 || batch < 2) return pl;  // no workspace: the other kernels need none
  const int units = w.cols / kSegCols;
  pl.row_groups = (w.rows + kSRows - 1) / kSRows;
  // activations of one slice must fit the LDS budget (60 KB, leaving room
  // for the kernel's static LDS under the 64 KB per-block default)
  int max_ups = ((60 * 1024 / 2) / batch - 8) / kSegCols / 4 * 4;
  if (max_ups > 4 * kSMaxBlocks) max_ups = 4 * kSMaxBlocks;  // every block's weights in registers
  if (max_ups < 4) max_ups = 4;
  // about one block per CU: 256 / row groups slices, at least 4 units each
  int ks = (256 + pl.row_groups - 1) / pl.row_groups;
  if (ks > (units + 3) / 4) ks = (units + 3) / 4;
  if (ks < 1) ks = 1;
  int ups = ((units + ks - 1) / ks + 3) / 4 * 4;
  if (ups > max_ups) ups = max_ups;
  pl.ups = ups;
  pl.ksplit = (units + ups - 1) / ups;
  // When the split pays: where the rows kernel does not fit (K > 32768), and
  // for K > 16384 at batch > 8 on at most 4096 rows.  Measured on MI355X: on
  // the 13B-shaped layers the rows kernel is as fast or faster at every batch
  // (5120x13824 at batch 16: 19.5 us both; everywhere else 5-40 % faster);
  // with four chunks per wave (K > 16384), hot, us at b4 / b8 / b16:
  // 4096x28672 rows 17.4 / 20.8 / 29.9 against split 23.3 / 23.1 / 24.7,
  // 8192x20480 rows 25.5 / 30.6 / 43.3 against split 47.3 / 47.5 / 46.6.
  // The rows kernel needs no workspace and no second launch.
  const bool wanted = units > 4 * kRMaxWaves * kRUnits ||
                      (units > 2 * kRMaxWaves * kRUnits && batch > 8 && w.rows <= 4096);
  if (!wanted) return SplitPlan{};
  if (pl.ksplit > 1) pl.partial_bytes = (size_t)pl.ksplit * pl.row_groups * kSWaves * kSTiles * kSPartialTileBytes;
  pl.workspace_bytes = pl.partial_bytes;
  return pl;
}

}  // namespace i4s
