// Batch SparseGEMV kernels for gfx950 (1 <= batch <= 16, and batch 1 for
// the 1:4 pattern) and the dispatch of every GEMV call.
//
// Method: "Efficient LLM-based Advertising via Model Compression and Parallel
// Verification", section 3.3, "Computational Acceleration" (activations
// staged on chip, INT4 widened in registers, 2-bit indices decoded with bit
// operations), and section 3.4, "Tree-based Parallel Verification", whose
// candidate sequences, decoded in parallel, make the batch of activation
// vectors.
//
// VALU batch kernel: a block is 4 waves; each wave owns RPW rows and the
// lanes take 64-column units as in the batch-1 kernels.  BT activation
// vectors (BT >= batch, rounded up to 1, 2, 4, 8, 16; the extra vectors are
// zero in LDS and never stored) are staged in LDS with 68 halfs per unit, so
// the 8-byte reads of 64 lanes fall in distinct banks.  When the staged
// activations exceed the LDS budget the K axis is processed in chunks.

#include "i4s_gemv_common.h"

namespace i4s {
namespace {

// ---------------------------------------------------------------------------
// batch kernel (any N, 1 <= batch <= 16)

// Accumulate one unit of RPW rows into acc[r][b].  xs points at the LDS copy
// of the unit's 64 columns for batch vector 0; vector b is xstride halfs on.
template <int NK, int BT, int RPW>
__device__ inline void compute_unit(const UnitRegs<NK> (&u)[RPW], const uint16_t *xs, int xstride,
                                    const uint32_t *lut, float (&acc)[RPW][BT]) {
  float g[RPW][BT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) g[r][b] = 0.0f;

  if constexpr (NK == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // vals word j = groups 4j..4j+3
      h2_t q[RPW][4];
#pragma unroll
      for (int r = 0; r < RPW; ++r) dequant_word(u[r].v[j], q[r]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int grp = 4 * j + p;
        uint2 xg[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) xg[b] = *reinterpret_cast<const uint2 *>(xs + b * xstride + 4 * grp);
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const uint32_t cw = u[r].c[j >> 1] >> (16 * (j & 1));
          const uint32_t sel = lut_read(lut, ((cw >> (4 * p)) & 0xFu) << 2);
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            const uint32_t xp = __builtin_amdgcn_perm(xg[b].y, xg[b].x, sel);
            g[r][b] = __builtin_amdgcn_fdot2(q[r][p], as_h2(xp), g[r][b], false);
          }
        }
      }
    }
  } else if constexpr (NK == 4) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // vals word j = columns 8j..8j+7
      h2_t q[RPW][4];
#pragma unroll
      for (int r = 0; r < RPW; ++r) dequant_word(u[r].v[j], q[r]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint2 xg[BT];
#pragma unroll
        for (int b = 0; b < BT; ++b) xg[b] = *reinterpret_cast<const uint2 *>(xs + b * xstride + 8 * j + 4 * h);
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            g[r][b] = __builtin_amdgcn_fdot2(q[r][2 * h], as_h2(xg[b].x), g[r][b], false);
            g[r][b] = __builtin_amdgcn_fdot2(q[r][2 * h + 1], as_h2(xg[b].y), g[r][b], false);
          }
      }
    }
  } else {  // NK == 1: element e of the unit is group e, column 4e + code
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      h2_t q[RPW][4];
#pragma unroll
      for (int r = 0; r < RPW; ++r) dequant_word(u[r].v[j], q[r]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e0 = 8 * j + 2 * p;  // elements e0 (group e0) and e0+1
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const uint32_t c0 = (u[r].c[0] >> (2 * e0)) & 3u;
          const uint32_t c1 = (u[r].c[0] >> (2 * e0 + 2)) & 3u;
#pragma unroll
          for (int b = 0; b < BT; ++b) {
            const uint32_t lo = xs[b * xstride + 4 * e0 + c0];
            const uint32_t hi = xs[b * xstride + 4 * e0 + 4 + c1];
            g[r][b] = __builtin_amdgcn_fdot2(q[r][p], as_h2(lo | (hi << 16)), g[r][b], false);
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float s = fp16_bits_to_float(u[r].s);
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[r][b] = fmaf(s, g[r][b], acc[r][b]);
  }
}

template <int NK, int BT, int RPW>
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    int rows, int cols, int group_size, const int32_t *__restrict__ row_ptr,
    const uint8_t *__restrict__ vals, const uint16_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x, int batch,
    uint16_t *__restrict__ y, int kc_units) {
  extern __shared__ __align__(16) uint16_t xs[];  // [BT][kc_units][kStrideBT]
  __shared__ uint32_t lut[16];
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int row0 = (blockIdx.x * kWaves + wave) * RPW;
  const int units = cols / kSegCols;
  const uint32_t nnz_row = (uint32_t)cols / 4 * NK;
  const int sg_shift = group_size == 64 ? 0 : (group_size == 128 ? 1 : 2);  // log2(G / 64)
  const uint32_t ngroups = (uint32_t)(cols / group_size);
  const int xstride = kc_units * kStrideBT;  // halfs between batch vectors in LDS

  // Rows past the end re-read the last row (their sums are never stored),
  // so every load and every decode below works on real data.
  uint32_t rstart[RPW], srow[RPW];
  bool rvalid[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    rvalid[r] = row0 + r < rows;
    const int rr = min(row0 + r, rows - 1);
    rstart[r] = (uint32_t)rr * nnz_row;  // the format's offset
    srow[r] = (uint32_t)rr * ngroups;    // first scale of the row
  }

  float acc[RPW][BT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[r][b] = 0.0f;

  for (int ub = 0; ub < units; ub += kc_units) {
    const int ue = min(units, ub + kc_units);
    int u = ub + lane;
    bool has = u < ue;
    UnitRegs<NK> cur[RPW];
    if (has) {
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        load_unit<NK>(cur[r], vals, codes, scales, rstart[r] + (uint32_t)u * 16 * NK,
                      srow[r] + ((uint32_t)u >> sg_shift));
    }
    int32_t rp[RPW];
    if (ub == 0) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) rp[r] = row_ptr[min(row0 + r, rows - 1)];
    }

    if (ub > 0) __syncthreads();  // the previous chunk is fully consumed
    {
      const int vpb = (ue - ub) * (kSegCols / 8);  // uint4 per batch vector
      for (int i = threadIdx.x; i < BT * vpb; i += kThreads) {
        const int b = i / vpb, c = i % vpb;
        const int un = c >> 3, part = c & 7;
        uint2 lo = make_uint2(0u, 0u), hi = make_uint2(0u, 0u);
        if (b < batch) {
          const uint4 v = *reinterpret_cast<const uint4 *>(x + (int64_t)b * cols + (int64_t)ub * kSegCols + 8 * c);
          lo = make_uint2(v.x, v.y);
          hi = make_uint2(v.z, v.w);
        }
        uint16_t *dst = xs + b * xstride + un * kStrideBT + 8 * part;  // 8-byte aligned
        reinterpret_cast<uint2 *>(dst)[0] = lo;
        reinterpret_cast<uint2 *>(dst)[1] = hi;
      }
      if (NK == 2 && ub == 0 && threadIdx.x < 16) init_selector_table(lut);
    }
    __syncthreads();

    if (ub == 0) {
      bool moved = false;
#pragma unroll
      for (int r = 0; r < RPW; ++r) moved |= (uint32_t)rp[r] != rstart[r];
      if (moved) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          rstart[r] = (uint32_t)rp[r];
          if (has)
            load_unit<NK>(cur[r], vals, codes, scales, rstart[r] + (uint32_t)u * 16 * NK,
                          srow[r] + ((uint32_t)u >> sg_shift));
        }
      }
    }

    while (has) {
      const int un = u + 64;
      const bool hn = un < ue;
      UnitRegs<NK> nxt[RPW];
      if (hn) {  // prefetch the lane's next unit
#pragma unroll
        for (int r = 0; r < RPW; ++r)
          load_unit<NK>(nxt[r], vals, codes, scales, rstart[r] + (uint32_t)un * 16 * NK,
                        srow[r] + ((uint32_t)un >> sg_shift));
      }
      compute_unit<NK, BT, RPW>(cur, xs + (u - ub) * kStrideBT, xstride, lut, acc);
      if (!hn) break;
#pragma unroll
      for (int r = 0; r < RPW; ++r) cur[r] = nxt[r];
      u = un;
    }
  }

#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const float t = wave_sum(acc[r][b]);
      if (lane == 0 && rvalid[r] && b < batch)
        y[(int64_t)b * rows + row0 + r] = (uint16_t)float_to_fp16_bits(t);
    }
}

// ---------------------------------------------------------------------------
// batch kernel on the sparse matrix cores (2:4, 2 <= batch <= 16)
//
// v_smfmac_f32_16x16x64_f16 multiplies a 16x64 2:4-sparse A (8 kept fp16
// values per lane plus their 2-bit in-group positions) by a dense 64x16 B
// and accumulates a 16x16 fp32 tile.  Here A is 16 weight rows and B is 64
// columns of the 16 activation vectors (vectors past `batch` are zero).  On
// gfx950 lane l = i + 16*kq of A holds row i's kept elements 8kq..8kq+7 of the
// tile's 64 columns, and its index VGPR holds their 2-bit positions at bits
// 2e (low half; abid 1 selects the high half) -- exactly one 32-bit vals word
// and one uint16 code word of the 2-bit CSR format, so the codes go to the
// matrix core untouched.  B lane j + 16*bq holds vector j's columns
// 8bq..8bq+7 and 32+8bq..32+8bq+7; the accumulator lane j + 16*q holds rows
// 4q..4q+3 of vector j.
//
// A lane loads one whole 64-column unit of its row (16-byte vals, 8-byte
// codes, its scale) for each block of 4 units; a 4x4 transpose across the 4
// lanes of a row (v_permlane32_swap + v_permlane16_swap) then hands lane kq
// word kq of each unit, so one matrix instruction covers exactly one unit,
// which lies in one quantization group: the group scale multiplies the fp32
// tile after the group's last unit (exact, as in the other kernels).  Scales
// move from the loading lanes to the accumulator lanes through a small
// wave-private LDS slot.
//
// A block is one 16-row tile and 8 waves; wave w takes blocks of 4 units
// w, w+8, ... (a K split inside the block) and reads its B fragments straight
// from global memory (x is small and stays in L2), so there is no block-wide
// staging and no barrier until the 8 partial tiles are summed in LDS at the
// end.  The next block's weights and activations are loaded while the
// current one runs on the matrix core.

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h16_t __attribute__((ext_vector_type(16)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u8_t __attribute__((ext_vector_type(8)));

constexpr int kMWaves = 8;

// Transpose a 4x4 block of dwords held by the 4 lanes i, i+16, i+32, i+48:
// on return lane-row q holds in v_s what lane-row s held in v_q.
__device__ inline void transpose4(uint32_t &v0, uint32_t &v1, uint32_t &v2, uint32_t &v3) {
  auto a = __builtin_amdgcn_permlane32_swap(v0, v2, false, false);
  v0 = a[0]; v2 = a[1];
  auto b = __builtin_amdgcn_permlane32_swap(v1, v3, false, false);
  v1 = b[0]; v3 = b[1];
  auto c = __builtin_amdgcn_permlane16_swap(v0, v1, false, false);
  v0 = c[0]; v1 = c[1];
  auto d = __builtin_amdgcn_permlane16_swap(v2, v3, false, false);
  v2 = d[0]; v3 = d[1];
}

// Codes of one unit per lane-row (c0 = halfwords 0,1; c1 = halfwords 2,3) ->
// p = (halfword q of unit 0, of unit 2), r = (halfword q of unit 1, of unit 3)
// for lane-row q.
__device__ inline void transpose_codes(uint32_t c0, uint32_t c1, uint32_t &p, uint32_t &r) {
  auto a = __builtin_amdgcn_permlane32_swap(c0, c1, false, false);
  const uint32_t lo = __builtin_amdgcn_perm(a[1], a[0], 0x05040100u);
  const uint32_t hi = __builtin_amdgcn_perm(a[1], a[0], 0x07060302u);
  auto b = __builtin_amdgcn_permlane16_swap(lo, hi, false, false);
  p = b[0];
  r = b[1];
}

template <int S>
__device__ inline f4_t smfmac_step(const uint32_t w, const h16_t &bx, const f4_t &c, uint32_t p, uint32_t r) {
  h2_t q[4];
  dequant_word(w, q);
  u4_t qa = {__builtin_bit_cast(uint32_t, q[0]), __builtin_bit_cast(uint32_t, q[1]),
             __builtin_bit_cast(uint32_t, q[2]), __builtin_bit_cast(uint32_t, q[3])};
  const h8_t a = __builtin_bit_cast(h8_t, qa);
  const int idx = (int)((S & 1) ? r : p);
  return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, bx, c, idx, 0, S >> 1);
}

// Registers of one block of 4 units for one lane.
struct MBlock {
  uint32_t v[4];   // vals words of the lane's unit
  uint32_t c[2];   // its code words
  uint32_t s;      // its scale
  uint4 x[8];      // B fragments of the 4 units (2 x 16 bytes each)
};


__global__ __launch_bounds__(64 * kMWaves) void gemv_smfmac_kernel(
    int rows, int cols, int group_size, const int32_t *__restrict__ row_ptr,
    const uint8_t *__restrict__ vals, const uint16_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x, int batch,
    uint16_t *__restrict__ y) {
  __shared__ __align__(16) uint16_t scs[kMWaves][4][16];   // per wave: scales of 4 units x 16 rows
  __shared__ __align__(16) float red[kMWaves][4][64];      // partial tiles
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int li = lane % 16, lq = lane / 16;
  const int row0 = blockIdx.x * 16;
  const int units = cols / kSegCols;
  const int nblk = (units + 3) / 4;
  const uint32_t nnz_row = (uint32_t)cols / 2;
  const int sg = group_size / kSegCols;
  const int sg_shift = sg == 1 ? 0 : (sg == 2 ? 1 : 2);
  const uint32_t ngroups = (uint32_t)(cols / group_size);

  // this lane's weight row (clamped: rows past the end re-read the last row)
  const int arow = min(row0 + li, rows - 1);
  uint32_t rstart = (uint32_t)arow * nnz_row;  // the format's offset; checked against row_ptr below
  // B lane (vector li, column quarter lq).  Lanes of vectors past `batch`
  // read the last real vector: B column j only feeds output column j, and
  // those columns are never stored.
  const uint16_t *xrow = x + (int64_t)min(li, batch - 1) * cols + 8 * lq;

  // Loads block b (units 4b..4b+3).  Units past the end re-read the last
  // unit; the matrix steps of those units are skipped, and the transposes
  // only move a unit's data into that unit's own step.
  auto load = [&](MBlock &m, int b) {
    const int u = min(4 * b + lq, units - 1);
    const uint32_t e0 = rstart + (uint32_t)u * 32;
    const uint4 v = *reinterpret_cast<const uint4 *>(vals + (e0 >> 1));
    const uint2 c = *reinterpret_cast<const uint2 *>(codes + (e0 >> 3));
    m.v[0] = v.x; m.v[1] = v.y; m.v[2] = v.z; m.v[3] = v.w;
    m.c[0] = c.x; m.c[1] = c.y;
    m.s = scales[(uint32_t)arow * ngroups + ((uint32_t)u >> sg_shift)];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int uu = min(4 * b + s, units - 1);
      m.x[2 * s] = *reinterpret_cast<const uint4 *>(xrow + uu * kSegCols);
      m.x[2 * s + 1] = *reinterpret_cast<const uint4 *>(xrow + uu * kSegCols + 32);
    }
  };

  f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto process = [&](const MBlock &m, int b) {
    uint32_t W0 = m.v[0], W1 = m.v[1], W2 = m.v[2], W3 = m.v[3], P, Q;
    transpose4(W0, W1, W2, W3);
    transpose_codes(m.c[0], m.c[1], P, Q);
    scs[wave][lq][li] = (uint16_t)m.s;  // scale of (row li, unit 4b+lq)
    f4_t cg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int u = 4 * b + s;
      if (u >= units) break;
      const u8_t xv = {m.x[2 * s].x, m.x[2 * s].y, m.x[2 * s].z, m.x[2 * s].w,
                       m.x[2 * s + 1].x, m.x[2 * s + 1].y, m.x[2 * s + 1].z, m.x[2 * s + 1].w};
      const h16_t bx = __builtin_bit_cast(h16_t, xv);
      if (s == 0) cg = smfmac_step<0>(W0, bx, cg, P, Q);
      if (s == 1) cg = smfmac_step<1>(W1, bx, cg, P, Q);
      if (s == 2) cg = smfmac_step<2>(W2, bx, cg, P, Q);
      if (s == 3) cg = smfmac_step<3>(W3, bx, cg, P, Q);
      if (((u + 1) & (sg - 1)) == 0) {  // the group ends with this unit
        const uint2 sv = *reinterpret_cast<const uint2 *>(&scs[wave][s][4 * lq]);
        acc[0] = fmaf(fp16_bits_to_float(sv.x & 0xFFFFu), cg[0], acc[0]);
        acc[1] = fmaf(fp16_bits_to_float(sv.x >> 16), cg[1], acc[1]);
        acc[2] = fmaf(fp16_bits_to_float(sv.y & 0xFFFFu), cg[2], acc[2]);
        acc[3] = fmaf(fp16_bits_to_float(sv.y >> 16), cg[3], acc[3]);
        cg = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  };

  int b = wave;
  MBlock ma, mb;
  if (b < nblk) {
    load(ma, b);
    const int32_t rp = row_ptr[arow];
    if ((uint32_t)rp != rstart) {  // a row stored elsewhere: re-fetch from row_ptr's offset
      rstart = (uint32_t)rp;
      load(ma, b);
    }
  }
  // two register sets in turn: the next block loads while the current runs
  while (b < nblk) {
    if (b + kMWaves < nblk) load(mb, b + kMWaves);
    process(ma, b);
    b += kMWaves;
    if (b >= nblk) break;
    if (b + kMWaves < nblk) load(ma, b + kMWaves);
    process(mb, b);
    b += kMWaves;
  }

  // sum the partial tiles of the 8 waves and store
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int l = threadIdx.x % 64, r = threadIdx.x / 64;
    float v = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kMWaves; ++wv) v += red[wv][r][l];
    const int j = l % 16, row = row0 + 4 * (l / 16) + r;
    if (j < batch && row < rows) y[(int64_t)j * rows + row] = (uint16_t)float_to_fp16_bits(v);
  }
}

// ---------------------------------------------------------------------------
// batch kernel on the sparse matrix cores with a K split across blocks
//
// Same matrix-core step as above, but a block owns 128 rows (8 waves x one
// 16-row tile) and one slice of K.  The slice of x (batch vectors x the
// slice's columns) is staged once in LDS and shared by the 8 tiles, so the
// activations cross from L2 once per 128 rows instead of once per 16.  Each
// block writes its 8 partial fp32 tiles to the caller's workspace; the block
// that finishes a row group last (a per-group counter in the workspace) sums
// the slices in slice order -- the result does not depend on which block is
// last -- stores y and resets the counter to zero for the next call.

constexpr int kSWaves = 8;              // tiles (waves) per block
constexpr int kSRows = 16 * kSWaves;    // rows per block
constexpr int kSMaxBlocks = 8;          // blocks of 4 units per slice (all loaded up front)

// Weight registers of one block of 4 units for one lane.
struct WBlock {
  uint32_t v[4];
  uint32_t c[2];
  uint32_t s;
};

__global__ __launch_bounds__(64 * kSWaves) void gemv_smfmac_split_kernel(
    int rows, int cols, int group_size, const int32_t *__restrict__ row_ptr,
    const uint8_t *__restrict__ vals, const uint16_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x, int batch,
    uint16_t *__restrict__ y, uint32_t *__restrict__ counters, f4_t *__restrict__ partial,
    int ksplit, int ups) {
  extern __shared__ __align__(16) uint16_t xs[];          // [batch][ups * 64 + 8]
  __shared__ __align__(16) uint16_t scs[kSWaves][4][16];
  __shared__ int last_block;
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int li = lane % 16, lq = lane / 16;
  const int rg = blockIdx.x, ks = blockIdx.y, ngrp = gridDim.x;
  const int row0 = rg * kSRows + 16 * wave;
  const int units = cols / kSegCols;
  const int u0 = ks * ups, u1 = min(units, u0 + ups);
  const int xst = ups * kSegCols + 8;  // halfs per vector in LDS (16-byte pad)
  const uint32_t nnz_row = (uint32_t)cols / 2;
  const int sg = group_size / kSegCols;
  const int sg_shift = sg == 1 ? 0 : (sg == 2 ? 1 : 2);
  const uint32_t ngroups = (uint32_t)(cols / group_size);

  const int arow = min(row0 + li, rows - 1);
  uint32_t rstart = (uint32_t)arow * nnz_row;
  // B lane (vector li, column quarter lq); lanes past `batch` read the last
  // real vector (their output columns are never stored)
  const uint16_t *xl = xs + min(li, batch - 1) * xst + 8 * lq;

  auto load = [&](WBlock &m, int b) {  // weights of block b (units 4b..4b+3) of this tile
    const int u = min(4 * b + lq, u1 - 1);
    const uint32_t e0 = rstart + (uint32_t)u * 32;
    const uint4 v = *reinterpret_cast<const uint4 *>(vals + (e0 >> 1));
    const uint2 c = *reinterpret_cast<const uint2 *>(codes + (e0 >> 3));
    m.v[0] = v.x; m.v[1] = v.y; m.v[2] = v.z; m.v[3] = v.w;
    m.c[0] = c.x; m.c[1] = c.y;
    m.s = scales[(uint32_t)arow * ngroups + ((uint32_t)u >> sg_shift)];
  };

  f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto process = [&](const WBlock &m, int b) {
    uint32_t W0 = m.v[0], W1 = m.v[1], W2 = m.v[2], W3 = m.v[3], P, Q;
    transpose4(W0, W1, W2, W3);
    transpose_codes(m.c[0], m.c[1], P, Q);
    scs[wave][lq][li] = (uint16_t)m.s;
    f4_t cg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int u = 4 * b + s;
      if (u >= u1) break;
      const uint4 xa = *reinterpret_cast<const uint4 *>(xl + (u - u0) * kSegCols);
      const uint4 xc = *reinterpret_cast<const uint4 *>(xl + (u - u0) * kSegCols + 32);
      const u8_t xv = {xa.x, xa.y, xa.z, xa.w, xc.x, xc.y, xc.z, xc.w};
      const h16_t bx = __builtin_bit_cast(h16_t, xv);
      if (s == 0) cg = smfmac_step<0>(W0, bx, cg, P, Q);
      if (s == 1) cg = smfmac_step<1>(W1, bx, cg, P, Q);
      if (s == 2) cg = smfmac_step<2>(W2, bx, cg, P, Q);
      if (s == 3) cg = smfmac_step<3>(W3, bx, cg, P, Q);
      if (((u + 1) & (sg - 1)) == 0) {
        const uint2 sv = *reinterpret_cast<const uint2 *>(&scs[wave][s][4 * lq]);
        acc[0] = fmaf(fp16_bits_to_float(sv.x & 0xFFFFu), cg[0], acc[0]);
        acc[1] = fmaf(fp16_bits_to_float(sv.x >> 16), cg[1], acc[1]);
        acc[2] = fmaf(fp16_bits_to_float(sv.y & 0xFFFFu), cg[2], acc[2]);
        acc[3] = fmaf(fp16_bits_to_float(sv.y >> 16), cg[3], acc[3]);
        cg = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  };

  // All of this tile's weights for the slice are requested at once, before
  // the activations are staged, so the memory latency is paid once.
  const int b0 = u0 / 4, nb = (u1 + 3) / 4 - b0;  // nb <= kSMaxBlocks
  WBlock mw[kSMaxBlocks];
#pragma unroll
  for (int i = 0; i < kSMaxBlocks; ++i)
    if (i < nb) load(mw[i], b0 + i);
  const int32_t rp = row_ptr[arow];
  {
    const int vpb = (u1 - u0) * (kSegCols / 8);  // uint4 per vector
    for (int i = threadIdx.x; i < batch * vpb; i += 64 * kSWaves) {
      const int bv = i / vpb, c = i % vpb;
      *reinterpret_cast<uint4 *>(xs + bv * xst + 8 * c) =
          *reinterpret_cast<const uint4 *>(x + (int64_t)bv * cols + (int64_t)u0 * kSegCols + 8 * c);
    }
  }
  if ((uint32_t)rp != rstart) {  // a row stored elsewhere: re-fetch from row_ptr's offset
    rstart = (uint32_t)rp;
#pragma unroll
    for (int i = 0; i < kSMaxBlocks; ++i)
      if (i < nb) load(mw[i], b0 + i);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSMaxBlocks; ++i)
    if (i < nb) process(mw[i], b0 + i);

  if (ksplit == 1) {  // no split: store directly
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * lq + r;
      if (li < batch && row < rows) y[(int64_t)li * rows + row] = (uint16_t)float_to_fp16_bits(acc[r]);
    }
    return;
  }
  // Partial tile -> workspace, then the last block of the row group sums.
  // The 8 XCDs' L2 caches are not coherent with each other, and a device-
  // scope fence would write back and invalidate the whole L2; instead every
  // access to the workspace is a device-scope atomic, performed at the
  // memory-side coherence point, and the counter is bumped only after this
  // block's partial stores have completed (s_waitcnt on outstanding stores,
  // then the block barrier).
  {
    float *dst = reinterpret_cast<float *>(partial + ((size_t)(ks * ngrp + rg) * kSWaves + wave) * 64 + lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) __hip_atomic_store(dst + r, acc[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // all of this wave's stores acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&counters[rg], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_block = old == (uint32_t)(ksplit - 1);
  }
  __syncthreads();
  if (!last_block) return;
  f4_t sum = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = 0; k < ksplit; ++k) {
    const float *src = reinterpret_cast<const float *>(partial + ((size_t)(k * ngrp + rg) * kSWaves + wave) * 64 + lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[r] += __hip_atomic_load(src + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + 4 * lq + r;
    if (li < batch && row < rows) y[(int64_t)li * rows + row] = (uint16_t)float_to_fp16_bits(sum[r]);
  }
  if (threadIdx.x == 0)  // ready for the next call
    __hip_atomic_store(&counters[rg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// dispatch

template <int NK, int BT, int RPW>
hipError_t launch_t(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                    hipStream_t stream) {
  const int units = w.cols / kSegCols;
  int kc = kLdsBudget / (BT * kStrideBT * 2);
  if (kc > units) kc = units;
  const size_t lds = (size_t)BT * kc * kStrideBT * 2;
  const int rows_per_block = kWaves * RPW;
  const dim3 grid((unsigned)((w.rows + rows_per_block - 1) / rows_per_block)), block(kThreads);
  hipLaunchKernelGGL((gemv_kernel<NK, BT, RPW>), grid, block, lds, stream, w.rows, w.cols,
                     w.group_size, w.row_ptr, w.vals, w.codes, w.scales, x, batch, y, kc);
  return hipGetLastError();
}

hipError_t launch_smfmac(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                         hipStream_t stream) {
  const dim3 grid((unsigned)((w.rows + 15) / 16)), block(64 * kMWaves);
  hipLaunchKernelGGL(gemv_smfmac_kernel, grid, block, 0, stream, w.rows, w.cols, w.group_size, w.row_ptr,
                     w.vals, w.codes, w.scales, x, batch, y);
  return hipGetLastError();
}

hipError_t launch_smfmac_split(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                               const SplitPlan &pl, void *workspace, hipStream_t stream) {
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  uint32_t *counters = reinterpret_cast<uint32_t *>(ws);
  f4_t *partial = reinterpret_cast<f4_t *>(ws + pl.counter_bytes);
  const size_t lds = (size_t)batch * (pl.ups * kSegCols + 8) * 2;
  const dim3 grid((unsigned)pl.row_groups, (unsigned)pl.ksplit), block(64 * kSWaves);
  hipLaunchKernelGGL(gemv_smfmac_split_kernel, grid, block, lds, stream, w.rows, w.cols, w.group_size,
                     w.row_ptr, w.vals, w.codes, w.scales, x, batch, y, counters, partial, pl.ksplit, pl.ups);
  return hipGetLastError();
}

// I4S_BATCH_PATH=valu forces the VALU batch kernel for 2:4 (tuning and
// cross-checks); read once.
bool smfmac_enabled() {
  static const bool v = [] {
    const char *e = getenv("I4S_BATCH_PATH");
    return !(e && e[0] == 'v');
  }();
  return v;
}

template <int NK>
hipError_t launch_nk(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                     hipStream_t stream) {
  if (NK == 2 && batch >= 2 && smfmac_enabled()) {
    return launch_smfmac(w, x, batch, y, stream);
  }
  if (batch <= 1) {
    if constexpr (NK == 2 || NK == 4) return launch_gemv_b1(w, x, y, stream);
    return launch_t<NK, 1, 4>(w, x, batch, y, stream);
  }
  if (batch <= 2) return launch_t<NK, 2, 4>(w, x, batch, y, stream);
  if (batch <= 4) return launch_t<NK, 4, 2>(w, x, batch, y, stream);
  if (batch <= 8) return launch_t<NK, 8, 2>(w, x, batch, y, stream);
  return launch_t<NK, 16, 1>(w, x, batch, y, stream);
}

}  // namespace

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
  // The split pays for its cross-block reduction (three dependent trips to
  // the memory-side coherence point, several microseconds) only when the
  // activations would otherwise cross from L2 once per 16 rows for many rows
  // or many columns: tall matrices, or wide ones at batch >= 8 (measured on
  // the 13B-shaped layers).  Otherwise the barrier-free kernel runs and no
  // workspace is needed.
  const bool worth_it = pl.row_groups >= 64 || (units >= 128 && batch >= 8);
  if (!worth_it || pl.row_groups > kSplitMaxRowGroups) return SplitPlan{};
  if (pl.ksplit > 1) {
    // The counters sit in a fixed region at the start of every workspace, so
    // layers of any shape that share a workspace never see each other's
    // partial tiles as counters; every completed call leaves that region zero.
    pl.counter_bytes = kSplitCounterBytes;
    pl.partial_bytes = (size_t)pl.ksplit * pl.row_groups * kSWaves * 64 * sizeof(float) * 4;
  }
  pl.workspace_bytes = pl.counter_bytes + pl.partial_bytes;
  return pl;
}

hipError_t launch_gemv_ws(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                          const SplitPlan &pl, void *workspace, hipStream_t stream) {
  if (pl.ksplit >= 1 && smfmac_enabled()) return launch_smfmac_split(w, x, batch, y, pl, workspace, stream);
  return launch_gemv(w, x, batch, y, stream);
}

hipError_t launch_gemv(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                       hipStream_t stream) {
  switch (w.n_keep) {
    case 1: return launch_nk<1>(w, x, batch, y, stream);
    case 2: return launch_nk<2>(w, x, batch, y, stream);
    default: return launch_nk<4>(w, x, batch, y, stream);
  }
}

}  // namespace i4s
