// Host-side plan of a GEMV call: whether the 2:4 batch GEMV splits K across
// blocks, and the workspace that needs (i4s_run_workspace_size, i4s_run_ws,
// i4s_run_noalloc).  Plain host code: no device code, no HIP calls.

#include "i4s_internal.h"

namespace i4s {

// Which batch 2:4 calls the K-split kernel takes (two launches: the sliced
// product, then the sum of the slices) rather than the rows kernel (one
// launch, every block over whole rows).  Measured on MI355X, cold, us per
// call, rows kernel against K split:
//   the rows kernel does not fit beyond K = 32768;
//   batch 3-8, long rows on few rows (the rows kernel then runs fewer than
//   ~190 blocks): 5120x13824 b3 / b4 / b8 14.7 / 14.9 / 16.1 against
//   14.4 / 14.3 / 14.4; 2048x8192 b8 8.0 / 6.9; 1024x16384 b4 10.4 / 8.1;
//   but 4096x11008 b4 (256 blocks) 10.8 / 11.3, 4096x14336 b6 11.4 / 12.2
//   and 5120x5120 b4 6.9 / 7.9; at batch 8 also 256 blocks: 4096x11008
//   12.2 / 10.6, 4096x14336 12.9 / 12.1, 4096x28672 22.4 / 19.1, 3072x8192
//   8.4 / 7.9 (8192x8192 11.5 / 11.7);
//   batch 9-16 on at most 512 tiles of 16 rows and K >= 5120: 5120x5120
//   9.5 / 8.3, 4096x11008 15.7 / 12.4, 4096x14336 17.3 / 13.4, 4096x28672
//   31.5 / 22.1, 8192x8192 13.7 / 13.4; but 4096x4096 6.7 / 7.3 and the
//   tall layers (13824x5120 13.3 / 15.5, 14336x4096 11.6 / 12.9);
//   batch 2: the rows kernel (5120x13824 14.5 / 14.8) or the VALU kernel.
bool split_wanted(int rows, int units, int32_t batch) {
  const int tiles = (rows + 15) / 16;
  if (units > 4 * kRMaxWaves * kRUnits) return true;  // K > 32768
  if (batch >= 3 && batch <= 8) {
    const int rows_blocks = tiles >= 300 ? (tiles + 1) / 2 : tiles;  // the rows kernel's blocks
    return units >= 128 && (rows_blocks < 192 || (batch == 8 && rows_blocks <= 256));
  }
  if (batch > 8) return units >= 80 && tiles <= 512;
  return false;
}

SplitPlan split_plan(const i4s_packed &w, int32_t batch) {
  SplitPlan pl{};
  if (w.n_keep != 2 || batch < 2) return pl;  // no workspace: the other kernels need none
  const int units = w.cols / kSegCols;
  if (!split_wanted(w.rows, units, batch)) return pl;
  const int tiles = (w.rows + 15) / 16;
  pl.ksplit = (units + kKUnits - 1) / kKUnits;
  // two tiles per wave above batch 8 where that still leaves >=
  // I4S_SPLIT_TW2_MIN_BLOCKS blocks, else one.  5120x13824, cold us, one /
  // two tiles: b4 12.24 / 13.25, b8 12.60 / 12.99, b16 14.75 / 14.28.
  const int groups2 = (tiles + 2 * kKWaves - 1) / (2 * kKWaves);
  pl.tw = batch > 8 && (int64_t)pl.ksplit * groups2 >= I4S_SPLIT_TW2_MIN_BLOCKS ? 2 : 1;
  pl.row_groups = (tiles + kKWaves * pl.tw - 1) / (kKWaves * pl.tw);
  if (pl.ksplit > 1)
    pl.partial_bytes = (size_t)pl.ksplit * pl.row_groups * kKWaves * pl.tw * kKPartialTileBytes;
  pl.workspace_bytes = pl.partial_bytes;
  return pl;
}

// Chunk width: 16 units (4 rows x 256 bytes per load) by default; 8 units
// (8 rows x 128 bytes, twice the waves per block, half the work each) when
// two-tile blocks are fewer than the compute units and the batch is at most
// 8.  Measured: 5120x5120 at batch 4 / 8 / 16: 7.45 / 7.76 / 8.90 us with 16,
// 6.63 / 7.32 / 9.01 with 8; 13824x5120 (432 blocks): 10.8 / 11.5 / 14.4 with
// 16, 11.6 / 12.9 / 16.5 with 8.
// want_u (8 or 16) fixes the chunk width; 0 chooses it.
RowsShape rows_shape(int units, int total_tiles, int batch, int n_keep, int want_u) {
  RowsShape r;
  // Four tiles per wave (8-unit chunks, one per wave) for batches above 8
  // on tall layers: each B fragment then feeds four tiles, halving the
  // activation reads through L2 against two tiles.  Cold, us at b16:
  // 13824x5120 15.4 -> 13.2, 11008x4096 12.0 -> 10.9; at b8 and below, and
  // with fewer than ~160 four-tile blocks, two tiles per wave are as fast or
  // faster (5120x5120 at b16: 9.1 against 12.0).  The block's LDS (waves x
  // 4 x 3.7 KB) caps K at 5632.  2:4 only: 1:4 on 11008x4096 at b12 / b16
  // took 12.37 / 12.83 us on four tiles, 11.46 / 12.18 on two tiles of
  // 16-unit chunks.
  const int tile8 = RowsGeom<8>::kTileLds;
  const bool four = n_keep == 2 && batch > 8 && total_tiles >= 640 && want_u != 16 &&
                    (size_t)((units + 7) / 8) * 4 * tile8 <= 160 * 1024;
  r.tpw = four ? 4 : (total_tiles >= 300 ? 2 : 1);
  r.u = ((r.tpw == 2 && total_tiles / 2 < 256 && batch <= 8) || r.tpw == 4) ? 8 : 16;
  // One-tile blocks, 1:4 in two-tile blocks, and two-tile blocks of rows of
  // at most 4096 columns, at batch <= 8: 8-unit chunks, twice the waves
  // (with the compact B fragments below where they fit), cold us at b4 / b8:
  // 4096x4096 1:4 4.74 / 5.15 -> 4.52 / 4.96 (per-lane fragments: 4.87 /
  // 5.42), 2:4 4.58 / 4.96 -> 4.45 / 4.89, dense 5.56 / 6.00 -> 5.49 / 5.67;
  // 11008x4096 1:4 10.07 / 10.90 -> 9.59 / 10.17 (per-lane fragments: 10.10
  // / 10.92), 2:4 9.09 / 9.90 -> 8.77 / 9.48, dense 12.96 / 13.59 -> 11.53 /
  // 13.05
  if ((r.tpw == 1 || n_keep == 1 || units <= 64) && r.tpw <= 2 && batch <= 8) r.u = 8;
  if (want_u) r.u = want_u;
  // 8-unit chunks only with one chunk per wave (K <= 8192): two chunks per
  // wave of the 16-wave form would not fit its 128 registers
  if ((units + 7) / 8 > RowsGeom<8>::kMaxWaves) r.u = 16;
  const int maxw = r.u == 8 ? RowsGeom<8>::kMaxWaves : RowsGeom<16>::kMaxWaves;
  const int chunks = (units + r.u - 1) / r.u;
  r.cpw = chunks > 2 * maxw ? 4 : (chunks > maxw ? 2 : 1);
  // dense rows are twice the bytes: two chunks of two tiles would spill; four
  // chunks per wave (K > 16384) always take one tile per wave
  if ((n_keep == 4 && r.cpw == 2) || r.cpw == 4) r.tpw = 1;
  // four tiles per wave: the 8-unit one-chunk form of 2:4 only (LDS)
  if (r.tpw == 4 && (r.u != 8 || r.cpw != 1 || n_keep != 2)) r.tpw = 2;
  r.waves = (chunks + r.cpw - 1) / r.cpw;
  const int tile_lds = n_keep == 4 ? (r.u == 8 ? RowsGeom<8, 4>::kTileLds : RowsGeom<16, 4>::kTileLds)
                                    : (r.u == 8 ? RowsGeom<8>::kTileLds : RowsGeom<16>::kTileLds);
  if (r.tpw == 4 && (size_t)r.waves * 4 * tile_lds > 160 * 1024) r.tpw = 2;  // LDS per workgroup
  r.lds = (size_t)r.waves * r.tpw * tile_lds;
  // At most four vectors (2:4 and dense): each wave reads a 4-unit block's
  // activations once (two 16-byte loads per lane instead of eight, three
  // quarters of which repeat the last vector) and spreads them through its
  // LDS area; measured cold, 13824x5120 at b4 11.4 -> 10.5 us, 5120x5120 at
  // b2 / b3 / b4 6.60 / 6.70 / 6.86 -> 6.29 / 6.38 / 6.43.  Not where the
  // extra LDS would exceed the workgroup limit, nor where it would leave
  // fewer blocks per CU on a layer with more blocks than the 256 CUs.
  // Five to eight vectors: four loads per lane and block, two passes through
  // the same area (two tiles of 16-unit chunks keep one block's loads in
  // flight instead of two, within their 128 registers): 5120x5120 at b8
  // 7.59 -> 6.96 us, 13824x5120 at b8 12.4 -> 11.9, 4096x4096 at b4 / b8
  // 4.87 / 5.49 -> 4.58 / 4.95, 4096x11008 (G64) at b4 10.69 -> 9.53.  1:4 only
  // with one 8-unit chunk per wave: with 16-unit chunks it came out 1-2 %
  // slower (4096x4096 1:4 at b4 / b8 4.75 / 5.15 -> 4.80 / 5.27).
  // Nine to sixteen vectors, one tile per wave: eight whole-row loads per
  // lane and block, four passes, one block ahead; at b12 / b16 on 4096x4096
  // 2:4 6.07 / 6.68 -> 5.53 / 5.54 us, dense 6.88 / 7.51 -> 6.61 / 6.64, 1:4
  // 5.74 / 6.31 -> 5.79 / 5.81 (with per-lane fragments each lane reads 16
  // bytes from each of two half rows).  The same on four-tile 2:4 blocks
  // where the LDS fits: 11008x4096 at b12 / b16 11.59 / 12.17 -> 11.36 /
  // 11.45; 1:4 there 12.36 / 12.83 -> 12.71 / 12.79, so not for 1:4.
  const int blocks = (total_tiles + r.tpw - 1) / r.tpw;
  const int want = batch <= 4 ? 4 : (batch <= 8 ? 8 : 16);
  const bool compact_ok = want == 16 ? (r.tpw == 1 || (r.tpw == 4 && n_keep == 2))
                                     : (r.tpw <= 2 && (n_keep != 1 || (r.u == 8 && r.cpw == 1)));
  if (compact_ok) {
    const size_t ldsc = r.lds + (size_t)r.waves * kRowsBcBytes;
    const size_t cu = 160 * 1024;
    if (ldsc <= cu && (cu / ldsc == cu / r.lds || blocks <= 256)) {
      r.bv = want;
      r.lds = ldsc;
    }
  }
  return r;
}

}  // namespace i4s
