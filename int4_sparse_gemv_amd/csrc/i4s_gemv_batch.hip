// Batch SparseGEMV kernels for gfx950 (2 <= batch <= 16) and the dispatch
// of every GEMV call.
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

#include <atomic>
#include <type_traits>

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
    // per row: the 8 element pairs' weights and selector pairs, then one
    // batch vector at a time (its 64 activations, 32 registers)
    h2_t q[RPW][8];
    u32x2_lut_t sel[RPW][8];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      dequant_word(u[r].v[0], &q[r][0]);
      dequant_word(u[r].v[1], &q[r][4]);
#pragma unroll
      for (int k = 0; k < 8; ++k) sel[r][k] = lut_read2(lut, ((u[r].c[0] >> (4 * k)) & 0xFu) << 3);
    }
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      uint2 xv[16];  // groups 0..15 of vector b
#pragma unroll
      for (int i = 0; i < 16; ++i) xv[i] = *reinterpret_cast<const uint2 *>(xs + b * xstride + 4 * i);
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t lo = __builtin_amdgcn_perm(xv[2 * k].y, xv[2 * k].x, sel[r][k].x);
          const uint32_t hi = __builtin_amdgcn_perm(xv[2 * k + 1].y, xv[2 * k + 1].x, sel[r][k].y);
          g[r][b] = __builtin_amdgcn_fdot2(q[r][k], as_h2(lo | hi), g[r][b], false);
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
  __shared__ __align__(8) uint32_t lut[32];
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
      if (ub == 0) init_tables<NK>(lut);
    }
    __syncthreads();

    if (ub == 0) {
      bool moved = false;
#pragma unroll
      for (int r = 0; r < RPW; ++r) moved |= (uint32_t)rp[r] != rstart[r];
      if (moved) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          rstart[r] = safe_row_start<NK>(rp[r], (uint32_t)(rows - 1) * nnz_row);
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
      // prefetch the lane's next unit; past the chunk's end the last unit is
      // read again and dropped.  Unconditional loads and a single exit at
      // the end keep the body one basic block: with a branch in the middle
      // the compiler hoisted every activation read of a unit ahead of its
      // dot products and spilled.
      const int uc = hn ? un : ue - 1;
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        load_unit<NK>(nxt[r], vals, codes, scales, rstart[r] + (uint32_t)uc * 16 * NK,
                      srow[r] + ((uint32_t)uc >> sg_shift));
      compute_unit<NK, BT, RPW>(cur, xs + (u - ub) * kStrideBT, xstride, lut, acc);
#pragma unroll
      for (int r = 0; r < RPW; ++r) cur[r] = nxt[r];
      u = un;
      has = hn;  // the only exit, at the end: the body stays one basic block
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
// wave-private LDS slot, with a wave-scope synchronisation on each side of
// the exchange (lanes read what other lanes of the wave wrote, and the slot
// is rewritten for the next block).  SG = G / 64 is a template parameter:
// blocks of 4 units start on multiples of 4, so where a group ends inside a
// block is known at compile time, and the block's scales are read before
// its matrix steps.
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


template <int SG>
__global__ __launch_bounds__(64 * kMWaves) void gemv_smfmac_kernel(
    int rows, int cols, const int32_t *__restrict__ row_ptr,
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
  constexpr int sg_shift = SG == 1 ? 0 : (SG == 2 ? 1 : 2);
  const uint32_t ngroups = (uint32_t)units >> sg_shift;

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
    wave_lds_sync();  // every lane has read the previous block's scales
    scs[wave][lq][li] = (uint16_t)m.s;  // scale of (row li, unit 4b+lq)
    wave_lds_sync();  // ... and the other lanes' writes are visible
    // the scales of the block's groups: rows 4lq..4lq+3 of each group's last unit
    uint2 sv[4 / SG];
#pragma unroll
    for (int g = 0; g < 4 / SG; ++g) sv[g] = *reinterpret_cast<const uint2 *>(&scs[wave][SG * g + SG - 1][4 * lq]);
    f4_t cg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int u = 4 * b + s;
      if (u >= units) break;  // units is a multiple of SG: the last unit ends a group
      const u8_t xv = {m.x[2 * s].x, m.x[2 * s].y, m.x[2 * s].z, m.x[2 * s].w,
                       m.x[2 * s + 1].x, m.x[2 * s + 1].y, m.x[2 * s + 1].z, m.x[2 * s + 1].w};
      const h16_t bx = __builtin_bit_cast(h16_t, xv);
      if (s == 0) cg = smfmac_step<0>(W0, bx, cg, P, Q);
      if (s == 1) cg = smfmac_step<1>(W1, bx, cg, P, Q);
      if (s == 2) cg = smfmac_step<2>(W2, bx, cg, P, Q);
      if (s == 3) cg = smfmac_step<3>(W3, bx, cg, P, Q);
      if ((s + 1) % SG == 0) {  // the group ends with this unit (4b is a multiple of SG)
        const uint2 g2 = sv[s / SG];
        acc[0] = fmaf(fp16_bits_to_float(g2.x & 0xFFFFu), cg[0], acc[0]);
        acc[1] = fmaf(fp16_bits_to_float(g2.x >> 16), cg[1], acc[1]);
        acc[2] = fmaf(fp16_bits_to_float(g2.y & 0xFFFFu), cg[2], acc[2]);
        acc[3] = fmaf(fp16_bits_to_float(g2.y >> 16), cg[3], acc[3]);
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
      rstart = safe_row_start<2>(rp, (uint32_t)(rows - 1) * nnz_row);
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
// batch kernel on the sparse matrix cores, one 16-row tile per block over the
// whole of K (2:4 and 1:4, 2 <= batch <= 16, K <= 16384; no workspace)
//
// How the weights of a tile are read decides the rate (measured on MI355X on
// a 13824x5120 layer): loads of 16 rows x 64 bytes per instruction -- the
// layout the matrix step wants -- stream at ~1.9 TB/s, while loads of 4 rows
// x 256 bytes per instruction, with each block covering whole rows, stream at
// ~4.9 TB/s, as fast as the batch-1 kernel's whole-row loads.  So each wave
// reads its 16-unit chunks of the tile's 16 rows in that shape (lane (u, r):
// row 4k + r, unit u), writes them to a wave-private LDS area and reads them
// back in the matrix layout (lane (i, kq): row i, unit 4b + kq), then goes
// on as the other SMFMAC kernels (4x4 transposes across the lane groups, one
// matrix step per unit, group scales on the fp32 tiles).  Only the wave
// itself touches its area, so no barrier is needed until the waves' partial
// tiles are summed in LDS at the end.  B fragments come from L2, two 4-unit
// blocks ahead of the matrix steps.
//
// 1:4 on the same matrix step: each group of 4 columns keeps one weight, so
// it is handed to the matrix core as a 2:4 group whose second kept value is
// zero -- positions (c & 2, (c & 2) + 1), the weight in slot c & 1 -- which
// is a canonical 2:4 group (two distinct ascending positions).  A unit is
// 8 bytes of vals and 4 bytes of codes; lane (row i, kq) reads its quarter
// (one half vals word, one code byte) straight from the wave's LDS area, so
// no transposes are needed.  The multiply count per unit is that of 2:4;
// the bytes are half.


// A dense unit-row: 64 nibbles, 32 bytes.
struct DenseVals {
  u32x4_t lo, hi;
};

constexpr int kRStride = kRUnits + 1;        // LDS row stride in elements (the wide form)
constexpr int kRValsBytes = RowsGeom<16>::kValsBytes;
constexpr int kRCodesBytes = RowsGeom<16>::kCodesBytes;
constexpr int kRWaveLds = RowsGeom<16>::kTileLds;  // 7040 bytes

// The matrix-step operands of one 1:4 unit for lane (row, kq): the unit's
// vals word kq / 2 and code byte kq (groups 4kq..4kq+3).  `sh` is 8 * (kq & 1):
// elements 4(kq & 1)..+3 of the word sit in nibble slots shifted by it.
__device__ inline f4_t smfmac_step_14(uint32_t wd, uint32_t cb, uint32_t sh, const h16_t &bx, const f4_t &c) {
  const uint32_t magic = 0x64006400u;
  const uint32_t t = wd >> sh;
  const h2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2_t bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  // (q_g0, q_g1) and (q_g2, q_g3) of the four groups
  const h2_t q01 = as_h2(and_or(t, 0x000F000Fu, magic)) + bias;
  const h2_t q23 = __builtin_elementwise_fma(as_h2(and_or(t, 0x00F000F0u, magic)), sixteenth, bias16);
  const uint32_t d01 = __builtin_bit_cast(uint32_t, q01), d23 = __builtin_bit_cast(uint32_t, q23);
  // group g's pair: its weight in slot (c_g & 1), a zero (selector byte
  // 0x0C) in the other; bit 2g of cb is c_g & 1
  const uint32_t b0 = cb & 1u, b1 = (cb >> 2) & 1u, b2 = (cb >> 4) & 1u, b3 = (cb >> 6) & 1u;
  u4_t qa;
  qa.x = __builtin_amdgcn_perm(0u, d01, 0x0C0C0100u ^ (b0 * 0x0D0C0D0Cu));
  qa.y = __builtin_amdgcn_perm(0u, d01, 0x0C0C0302u ^ (b1 * 0x0F0E0F0Eu));
  qa.z = __builtin_amdgcn_perm(0u, d23, 0x0C0C0100u ^ (b2 * 0x0D0C0D0Cu));
  qa.w = __builtin_amdgcn_perm(0u, d23, 0x0C0C0302u ^ (b3 * 0x0F0E0F0Eu));
  // positions: nibble g = (c_g & 2) | ((c_g & 2) + 1) << 2
  uint32_t y = cb;
  y = (y | (y << 4)) & 0x0F0Fu;  // codes 0,1 in byte 0, codes 2,3 in byte 1
  y = (y | (y << 2)) & 0x3333u;  // code g in bits 4g..4g+1
  const uint32_t idx = (y & 0x2222u) * 5u + 0x4444u;
  const h8_t a = __builtin_bit_cast(h8_t, qa);
  return __builtin_amdgcn_smfmac_f32_16x16x64_f16(a, bx, c, (int)idx, 0, 0);
}

// NK = 2 (2:4) or 1 (1:4).  CPW = 16-unit chunks per wave; waves per block =
// ceil(units / (16 * CPW)).  SG = units per quantization group (G / 64: 1, 2
// or 4), so where a group ends inside a block of 4 units is known at compile
// time.
// `blk` is the block's index within its layer: it covers the TPW 16-row
// tiles from row 16 * TPW * blk.  lds is the block's dynamic LDS (per wave:
// [TPW][RowsGeom<U>::kTileLds], then kRowsBcBytes when BV > 0).  Each B
// fragment a wave loads feeds the matrix steps of its TPW tiles (measured on
// the 13824x5120 layer: the B-fragment loads from L2, not the weight stream,
// bound the one-tile form; two tiles per wave take 14.8 -> 10.6 us at batch
// 4 and 23.4 -> 14.6 us at batch 16).
// BV = 4, 8 or 16 (at most that many vectors): a wave reads each 4-unit
// block's activations once, BV / 2 16-byte loads per lane in whole 128-byte
// rows, and spreads them to the matrix layout through kRowsBcBytes of its
// LDS area (in BV / 4 passes); BV = 0: every lane loads its own B fragment,
// 16 bytes from each of two half rows (at batch 4 three quarters of those
// bytes repeat the last vector, and all of them share the CU's vector
// memory path with the weight stream).
template <int NK, int CPW, int SG, int TPW, int U, int BV>
__device__ __forceinline__ void rows_body(
    int blk, int rows, int units, int sg_shift, const int32_t *__restrict__ row_ptr,
    const uint8_t *__restrict__ vals, const uint16_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x, int batch,
    uint16_t *__restrict__ y, uint8_t *lds) {
  typedef RowsGeom<U, NK> Geo;
  constexpr int RL = Geo::kRowsPerLoad, NL = Geo::kLoads, NBK = Geo::kBlocks, ST = Geo::kStride;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, nwaves = blockDim.x / 64;
  const int li = lane % 16, lq = lane / 16;  // the matrix layout
  const int lu = lane % U, lr = lane / U;     // the load layout: unit lu of row RL * k + lr
  const int row0 = blk * 16 * TPW;
  const uint32_t nnz_row = (uint32_t)units * 16 * NK;
  const uint32_t ngroups = (uint32_t)units >> sg_shift;
  // a unit-row's vals (dense: two 16-byte halves) and codes (none when dense)
  typedef typename std::conditional<NK == 4, DenseVals,
                                    typename std::conditional<NK == 2, u32x4_t, u32x2_t>::type>::type vals_t;
  typedef typename std::conditional<NK == 2, u32x2_t, uint32_t>::type codes_t;
  static_assert(BV == 0 || BV == 4 || BV == 8 || BV == 16, "B fragments: compact (4, 8, 16 vectors) or per lane");
  constexpr bool kCompact = BV > 0;
  constexpr int NI = kCompact ? BV / 2 : 1;  // compact loads per lane and 4-unit block
  constexpr int NP = kCompact ? BV / 4 : 1;  // passes through the LDS area per block
  constexpr int kWaveLds = TPW * Geo::kTileLds + (kCompact ? kRowsBcBytes : 0);
  uint8_t *wl = lds + wave * kWaveLds;  // the wave's areas: one per tile, then the activations' (BV > 0)
  uint8_t *wbc = wl + TPW * Geo::kTileLds;
  auto lv_of = [&](int t) { return reinterpret_cast<vals_t *>(wl + t * Geo::kTileLds); };  // [16 rows][ST]
  auto lc_of = [&](int t) { return reinterpret_cast<codes_t *>(wl + t * Geo::kTileLds + Geo::kValsBytes); };
  auto lsc_of = [&](int t) {                                                     // [U units][Geo::kScaleStride]
    return reinterpret_cast<uint16_t *>(wl + t * Geo::kTileLds + Geo::kValsBytes + Geo::kCodesBytes);
  };

  // B fragments: lane (vector li, column quarter lq); vectors past `batch`
  // read the last real one (their output columns are never stored).  Block
  // n of the wave = units 4n..4n+3 of its chunks, in order.
  const int cols = units * kSegCols;
  const uint16_t *xrow = x + (int64_t)min(li, batch - 1) * cols + 8 * lq;
  auto unit_of = [&](int n, int s) { return (wave * CPW + n / NBK) * U + 4 * (n % NBK) + s; };
  auto load_b = [&](u32x4_t (&bx)[8], int n) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int u = min(unit_of(n, s), units - 1);
      bx[2 * s] = *reinterpret_cast<const u32x4_t *>(xrow + u * kSegCols);
      bx[2 * s + 1] = *reinterpret_cast<const u32x4_t *>(xrow + u * kSegCols + 32);
    }
  };

  // every weight load of the wave: lane (unit lu, row lr): row 16t + RL k + lr
  int wrow[TPW][NL];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int k = 0; k < NL; ++k) wrow[t][k] = min(row0 + 16 * t + RL * k + lr, rows - 1);
  // BV > 0: load i of lane L takes piece (L % 8) ^ g(v) of the 128-byte
  // activation row of pair P = 8i + L / 8 (vector v = P % BV, unit P / BV of
  // the block), so every 8 lanes read one whole row.  A pass through the
  // wave's 2 KB area writes two loads in lane order (16 pairs: four units of
  // four vectors, two of eight or one of sixteen) and reads them back: lane (vector
  // li, quarter lq) takes pieces lq and 4 + lq of vector min(li, BV - 1) for
  // each unit of the pass.  g(v) = 4 for vectors 2, 3 (6, 7) moves their
  // pieces to the other half of the 128 bytes, so the distinct 16-byte reads
  // of one LDS instruction fall in distinct banks (BV = 4) or at most two to
  // a bank (BV = 8).
  constexpr int BVS = kCompact ? BV : 1;  // (the lambdas below are not called when BV = 0)
  auto swz = [](int v) { return 4 * ((v >> 1) & 1); };
  auto load_bc = [&](u32x4_t (&bc)[NI], int n) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int P = 8 * i + lane / 8, v = P % BVS, s = P / BVS;
      const int q = (lane % 8) ^ swz(v);
      const int u = min(unit_of(n, s), units - 1);
      bc[i] = *reinterpret_cast<const u32x4_t *>(x + (int64_t)min(v, batch - 1) * cols + u * kSegCols + 8 * q);
    }
  };
  // the B fragments of the pass's units (4 / NP of them, from unit s0) out of the area
  auto read_bc = [&](u32x4_t (&bx)[8], int s0) {
    const int v = min(li, BVS - 1), f = swz(v);
#pragma unroll
    for (int s = 0; s < 4 / NP; ++s) {
      const u32x4_t *a = reinterpret_cast<const u32x4_t *>(wbc) + (s * BVS + v) * 8;
      bx[2 * (s0 + s)] = a[lq ^ f];
      bx[2 * (s0 + s) + 1] = a[(4 + lq) ^ f];
    }
  };
  u32x4_t bq[2][8];   // BV = 0: the B fragments of blocks n and n + 1
  // BV > 0: the compact loads of blocks n and n + 1 (NBUF = 2), or of block
  // n alone, reloaded as soon as it sits in LDS (NBUF = 1: sixteen vectors,
  // and eight on two tiles of 16-unit chunks, whose two buffers would spill
  // at the 128-register cap)
  constexpr int NBUF = (BV == 16 || (BV == 8 && TPW == 2 && U == 16)) ? 1 : 2;
  u32x4_t bqc[NBUF][NI];
  if constexpr (kCompact) {
    load_bc(bqc[0], 0);
    if constexpr (NBUF == 2) load_bc(bqc[1], 1);
  } else {
    load_b(bq[0], 0);
    load_b(bq[1], 1);
  }
  vals_t wv[TPW][NL];  // one chunk; the next chunk reuses them once it is staged
  codes_t wc[TPW][NL];
  uint16_t wsc[TPW][NL];
  // The weights are fetched at the format's offsets (row * K * N / 4)
  // without waiting for row_ptr, which is read last and checked after the
  // pass.  The pass uses these loads on every path, so the compiler cannot
  // sink them below the check (an earlier arrangement that reloaded into the
  // same registers when a row had moved let it do exactly that, and the
  // weight stream then waited for row_ptr).
  // One chunk's weights at a time (two chunks at once would also exceed the
  // 63 vector loads a wave can have in flight): the next chunk is loaded
  // into the same registers as soon as the current one sits in LDS, and
  // streams in while it is multiplied.
  auto load_chunk = [&](int c) {
    const int u = min((wave * CPW + c) * U + lu, units - 1);
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int k = 0; k < NL; ++k) {
        const uint32_t e0 = (uint32_t)wrow[t][k] * nnz_row + (uint32_t)u * 16 * NK;
        const uint32_t si = (uint32_t)wrow[t][k] * ngroups + ((uint32_t)u >> sg_shift);
        if constexpr (NK == 4) {
          const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(vals + (e0 >> 1));
          wv[t][k].lo = __builtin_nontemporal_load(vp);
          wv[t][k].hi = __builtin_nontemporal_load(vp + 1);
        } else {
          wv[t][k] = __builtin_nontemporal_load(reinterpret_cast<const vals_t *>(vals + (e0 >> 1)));
          wc[t][k] = __builtin_nontemporal_load(reinterpret_cast<const codes_t *>(codes + (e0 >> 3)));
        }
        wsc[t][k] = __builtin_nontemporal_load(scales + si);
      }
  };
  load_chunk(0);
  int32_t rp[TPW][NL];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int k = 0; k < NL; ++k) rp[t][k] = row_ptr[wrow[t][k]];

  // one pass over the wave's chunks; B fragments two blocks ahead
  f4_t acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  {
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      // chunk c of every tile to the wave's LDS areas, in the load layout.
      // A unit past the row's end (only a row's last chunk can hold one; its
      // lane read the last unit again) must add nothing: its scale is staged
      // as +0, and since its unit never shares a quantization group with a
      // real one (K % G == 0), the group's partial tile (finite: real
      // nibbles and activations of the last unit) is multiplied by zero.
      // Only a value depends on the lane, so the loads are used on every
      // path and stay where they were issued; and there is no branch (even a
      // wave-uniform one here split the body and made the compiler spill).
      const bool unit_ok = (wave * CPW + c) * U + lu < units;
      // The area is the wave's own, written in the load layout and read back
      // by other lanes of the wave in the matrix layout: a wave-scope
      // synchronisation before the writes of every chunk after the first
      // (the previous chunk's reads are done) and after the writes (they are
      // visible).  The first chunk's area has not been read yet, and a
      // synchronisation there would also keep the compiler from issuing the
      // last weight and activation loads between the first LDS writes.
      if (c > 0) wave_lds_sync();
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        vals_t *lv = lv_of(t);
        codes_t *lc = lc_of(t);
        uint16_t *lsc = lsc_of(t);
#pragma unroll
        for (int k = 0; k < NL; ++k) {
          lv[(RL * k + lr) * ST + lu] = wv[t][k];
          if constexpr (NK != 4) lc[(RL * k + lr) * ST + lu] = wc[t][k];
          lsc[lu * Geo::kScaleStride + RL * k + lr] = unit_ok ? wsc[t][k] : (uint16_t)0;
        }
      }
      wave_lds_sync();
      if (c + 1 < CPW) {
        __builtin_amdgcn_sched_barrier(0);
        load_chunk(c + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int bb = 0; bb < NBK; ++bb) {
        const int n = NBK * c + bb;
        // BV > 0: block n's activations through the wave's area, NP passes
        // of two loads (each written once the previous pass's reads are done)
        u32x4_t bxl[8];
        if constexpr (kCompact) {
#pragma unroll
          for (int j = 0; j < NP; ++j) {
            if (n > 0 || j > 0) wave_lds_sync();
            reinterpret_cast<u32x4_t *>(wbc)[lane] = bqc[n % NBUF][2 * j];
            reinterpret_cast<u32x4_t *>(wbc)[64 + lane] = bqc[n % NBUF][2 * j + 1];
            wave_lds_sync();
            read_bc(bxl, j * (4 / NP));
          }
          if constexpr (NBUF == 1) {
            __builtin_amdgcn_sched_barrier(0);
            if (n + 1 < NBK * CPW) load_bc(bqc[0], n + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        u32x4_t (&bx)[8] = kCompact ? bxl : bq[n % 2];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const vals_t *lv = lv_of(t);
          const codes_t *lc = lc_of(t);
          const uint16_t *lsc = lsc_of(t);
          uint32_t W0 = 0, W1 = 0, W2 = 0, W3 = 0, P = 0, Q = 0;
          if constexpr (NK == 4) {
            // read per unit below (two words per lane and unit)
          } else if constexpr (NK == 2) {
            // the matrix layout: lane (row li, chunk lq) takes unit 4bb + lq
            const u32x4_t v = lv[li * ST + 4 * bb + lq];
            const u32x2_t cw = lc[li * ST + 4 * bb + lq];
            W0 = v.x; W1 = v.y; W2 = v.z; W3 = v.w;
            transpose4(W0, W1, W2, W3);
            transpose_codes(cw.x, cw.y, P, Q);
          } else {
            // lane (row li, quarter lq) of unit 4bb + s: vals word lq / 2 and
            // code byte lq, read in place
            const uint32_t *lvw = reinterpret_cast<const uint32_t *>(lv);
            const uint8_t *lcb = reinterpret_cast<const uint8_t *>(lc);
            const int e = li * ST + 4 * bb;
            W0 = lvw[2 * e + (lq >> 1)]; W1 = lvw[2 * (e + 1) + (lq >> 1)];
            W2 = lvw[2 * (e + 2) + (lq >> 1)]; W3 = lvw[2 * (e + 3) + (lq >> 1)];
            P = (uint32_t)lcb[4 * e + lq] | ((uint32_t)lcb[4 * (e + 1) + lq] << 8) |
                ((uint32_t)lcb[4 * (e + 2) + lq] << 16) | ((uint32_t)lcb[4 * (e + 3) + lq] << 24);
          }
          // the scales of the block's groups (rows 4lq..4lq+3 of each group's
          // last unit), read before the matrix steps
          u32x2_t sv[4 / SG];
#pragma unroll
          for (int g = 0; g < 4 / SG; ++g)
            sv[g] = *reinterpret_cast<const u32x2_t *>(&lsc[(4 * bb + SG * g + SG - 1) * Geo::kScaleStride + 4 * lq]);
          f4_t cg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const u8_t xv = {bx[2 * s].x, bx[2 * s].y, bx[2 * s].z, bx[2 * s].w,
                             bx[2 * s + 1].x, bx[2 * s + 1].y, bx[2 * s + 1].z, bx[2 * s + 1].w};
            const h16_t hb = __builtin_bit_cast(h16_t, xv);
            if constexpr (NK == 4) {
              // dense: two 16x16x32 steps per unit; lane (row li, quarter lq)
              // takes vals words lq and 4 + lq (columns 8lq.. and 32 + 8lq..)
              // of its row's unit, the B fragment's two halves are exactly
              // those columns of the vectors
              const uint32_t *lvw = reinterpret_cast<const uint32_t *>(lv);
              const int e = (li * ST + 4 * bb + s) * 8;
              h2_t qa[4], qb[4];
              dequant_word(lvw[e + lq], qa);
              dequant_word(lvw[e + 4 + lq], qb);
              const h8_t a0 = {qa[0].x, qa[0].y, qa[1].x, qa[1].y, qa[2].x, qa[2].y, qa[3].x, qa[3].y};
              const h8_t a1 = {qb[0].x, qb[0].y, qb[1].x, qb[1].y, qb[2].x, qb[2].y, qb[3].x, qb[3].y};
              cg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, __builtin_bit_cast(h8_t, bx[2 * s]), cg, 0, 0, 0);
              cg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, __builtin_bit_cast(h8_t, bx[2 * s + 1]), cg, 0, 0, 0);
            } else if constexpr (NK == 2) {
              if (s == 0) cg = smfmac_step<0>(W0, hb, cg, P, Q);
              if (s == 1) cg = smfmac_step<1>(W1, hb, cg, P, Q);
              if (s == 2) cg = smfmac_step<2>(W2, hb, cg, P, Q);
              if (s == 3) cg = smfmac_step<3>(W3, hb, cg, P, Q);
            } else {
              const uint32_t sh = 8u * (uint32_t)(lq & 1);
              const uint32_t wd = s == 0 ? W0 : (s == 1 ? W1 : (s == 2 ? W2 : W3));
              cg = smfmac_step_14(wd, (P >> (8 * s)) & 0xFFu, sh, hb, cg);
            }
            if ((s + 1) % SG == 0) {  // the group ends with this unit (chunks start on 4-unit bounds)
              const u32x2_t g2 = sv[s / SG];
              acc[t][0] = fmaf(fp16_bits_to_float(g2.x & 0xFFFFu), cg[0], acc[t][0]);
              acc[t][1] = fmaf(fp16_bits_to_float(g2.x >> 16), cg[1], acc[t][1]);
              acc[t][2] = fmaf(fp16_bits_to_float(g2.y & 0xFFFFu), cg[2], acc[t][2]);
              acc[t][3] = fmaf(fp16_bits_to_float(g2.y >> 16), cg[3], acc[t][3]);
              cg = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
          }
        }
        // the buffer just used takes block n + 2; the scheduling barriers keep
        // the loads here, so only two buffers are ever live
        __builtin_amdgcn_sched_barrier(0);
        if (n + 2 < NBK * CPW) {
          if constexpr (kCompact) {
            if constexpr (NBUF == 2) load_bc(bqc[n % 2], n + 2);
          } else {
            load_b(bx, n + 2);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // row_ptr check (wave-uniform; every wave of the block sees the same
  // rows).  A row stored away from the format's offset is rare: the wave
  // then recomputes its share of every tile from row_ptr's offsets with a
  // plain per-lane loop (lane (vector li, quarter lq) owns rows 4lq..4lq+3 of
  // each tile, as in the matrix accumulator), within the same tolerance.
  bool moved = false;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int k = 0; k < NL; ++k) moved |= (uint32_t)rp[t][k] != (uint32_t)wrow[t][k] * nnz_row;
  if (__builtin_amdgcn_ballot_w64(moved) != 0) {
    const uint16_t *xv = x + (int64_t)min(li, batch - 1) * cols;
    for (int t = 0; t < TPW; ++t) {
      for (int r = 0; r < 4; ++r) {
        const int row = min(row0 + 16 * t + 4 * lq + r, rows - 1);
        const uint32_t rs = safe_row_start<NK>(row_ptr[row], (uint32_t)(rows - 1) * nnz_row);
        float sum = 0.0f;
        for (int c = 0; c < CPW; ++c) {
          for (int uu = 0; uu < U; ++uu) {
            const int u = (wave * CPW + c) * U + uu;
            if (u >= units) break;
            float g = 0.0f;
            for (int e = 0; e < 16 * NK; ++e) {
              const uint32_t el = rs + (uint32_t)u * 16 * NK + (uint32_t)e;
              const uint32_t word = reinterpret_cast<const uint32_t *>(vals)[el >> 3];
              const uint32_t k8 = el & 7u;
              const uint32_t slot = (k8 & 1u) ? 4u + (k8 >> 1) : (k8 >> 1);
              const int q = (int)((word >> (4 * slot)) & 0xFu) - 8;
              const uint32_t code = NK == 4 ? (uint32_t)(e & 3) : (codes[el >> 3] >> (2 * (el & 7u))) & 3u;
              const int col = u * kSegCols + 4 * (e / NK) + (int)code;
              g = fmaf((float)q, fp16_bits_to_float(xv[col]), g);
            }
            sum = fmaf(fp16_bits_to_float(scales[(uint32_t)row * ngroups + ((uint32_t)u >> sg_shift)]), g, sum);
          }
        }
        acc[t][r] = sum;
      }
    }
  }

  // sum the waves' partial tiles (each wave writes into its own area, once
  // all its lanes are done reading it) and store y
  wave_lds_sync();
  f4_t *red = reinterpret_cast<f4_t *>(wl);
#pragma unroll
  for (int t = 0; t < TPW; ++t) red[64 * t + lane] = acc[t];
  lds_barrier();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      f4_t sum = acc[t];
      for (int w = 1; w < nwaves; ++w)
        sum += reinterpret_cast<const f4_t *>(lds + w * kWaveLds)[64 * t + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + 16 * t + 4 * lq + r;
        if (li < batch && row < rows) y[(int64_t)li * rows + row] = (uint16_t)float_to_fp16_bits(sum[r]);
      }
    }
  }
}

// Waves per SIMD the compiler must leave room for: the one-chunk two-tile
// 2:4 form runs two 8-wave blocks per CU only at <= 128 VGPRs (4 waves per
// SIMD); at 129 or more the blocks of a layer run one after the other.
template <int NK, int CPW, int TPW, int U>
constexpr int rows_min_waves() {
  return (NK == 2 && CPW == 1 && TPW == 2 && U == 16) ? 4 : 1;
}

template <int NK, int CPW, int SG, int TPW, int U, int BV>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 64 * (TPW == 4 ? 12 : RowsGeom<U>::kMaxWaves)),
                          amdgpu_waves_per_eu(rows_min_waves<NK, CPW, TPW, U>())))
void gemv_smfmac_rows_kernel(
    int rows, int units, int sg_shift, const int32_t *__restrict__ row_ptr,
    const uint8_t *__restrict__ vals, const uint16_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x, int batch,
    uint16_t *__restrict__ y) {
  extern __shared__ __align__(16) uint8_t lds[];  // [waves][TPW][RowsGeom<U>::kTileLds]
  rows_body<NK, CPW, SG, TPW, U, BV>(blockIdx.x, rows, units, sg_shift, row_ptr, vals, codes, scales, x, batch, y,
                                     lds);
}

// Several layers that share x (and N, G and K) in one launch: each block
// finds its layer from the cumulative block counts and runs the single-layer
// body on it.
template <int NK, int CPW, int SG, int TPW, int U, int BV>
__global__ __attribute__((amdgpu_flat_work_group_size(1, 64 * (TPW == 4 ? 12 : RowsGeom<U>::kMaxWaves)),
                          amdgpu_waves_per_eu(rows_min_waves<NK, CPW, TPW, U>())))
void gemv_smfmac_rows_multi_kernel(
    int units, const uint16_t *__restrict__ x, int batch, MultiDesc d) {
  extern __shared__ __align__(16) uint8_t lds[];  // [waves][TPW][RowsGeom<U>::kTileLds]
  int m = 0;
#pragma unroll
  for (int i = 1; i < kMaxMulti; ++i) m += (i < d.n && (int)blockIdx.x >= d.block_end[i - 1]) ? 1 : 0;
  const int first = m == 0 ? 0 : d.block_end[m - 1];
  rows_body<NK, CPW, SG, TPW, U, BV>((int)blockIdx.x - first, d.rows[m], units, d.sg_shift[m], d.row_ptr[m],
                                 d.vals[m], d.codes[m], d.scales[m], x, batch, d.y[m], lds);
}

// ---------------------------------------------------------------------------
// batch kernel on the sparse matrix cores with K split across blocks (2:4,
// 2 <= batch <= 16; needs the caller's workspace)
//
// A block is kKWaves waves, one slice of K (kKUnits = 16 units, 1024
// columns) and one group of kKWaves * TW 16-row tiles.  The slice is the fast
// block index, so the slices of a row group are in flight together and the
// group's rows are read as a whole.  The block stages its slice of x (the
// batch vectors' 1024 columns, rows padded by 16 bytes so that the B reads
// of 16 vectors fall in distinct banks) in LDS once; B fragments then come
// from LDS, not through the vector L1, which on this part moves ~56 bytes
// per clock per CU against several times that for LDS reads -- and a B
// fragment is 2 KB per unit whatever the batch, 5x the weight bytes of a
// tile's unit.  Each wave runs its TW tiles one after the other: it loads a
// tile's weights as 4 rows x 256 bytes per instruction (the shape that
// streams fastest), writes them to its LDS area in that layout, reads them
// back in the matrix layout (lane (i, kq): row i, unit 4b + kq) and goes on
// as the other SMFMAC kernels (4x4 transposes across the lane groups, one
// matrix step per unit, group scales on the fp32 tiles).  The loads of the
// next two tiles are in flight while a tile is multiplied.  Each tile's fp32
// partial product goes to the workspace, and a second small kernel sums the
// slices in slice order (deterministic) and stores y; the kernel boundary
// makes the partials visible across the XCDs' L2 caches, so no device-scope
// atomics, fences or counters are needed and the workspace is plain scratch.
// With a single slice (K <= 1024) the kernel stores y itself.

// partial tile index: slice ks, row group rg (of tpg tiles), tile t of the
// group; each tile is 64 lanes x 4 floats (lane j + 16q: rows 4q..4q+3,
// vector j)
__device__ inline size_t slice_tile(int ks, int ngrp, int rg, int tpg, int t) {
  return ((size_t)ks * ngrp + rg) * tpg + t;
}

// One tile's result of the slice kernel: y itself when there is a single
// slice, else the tile's partial (the columns of real vectors only).
__device__ inline void slice_store(const f4_t &acc, int tile, int ks, int ksplit, int rg, int ngrp, int tw,
                                   int rows, int batch, uint16_t *__restrict__ y, f4_t *__restrict__ partial) {
  const int lane = threadIdx.x % 64, li = lane % 16, lq = lane / 16;
  if (li >= batch) return;
  if (ksplit == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = tile * 16 + 4 * lq + r;
      if (row < rows) y[(int64_t)li * rows + row] = (uint16_t)float_to_fp16_bits(acc[r]);
    }
  } else {
    const int tpg = kKWaves * tw;
    partial[slice_tile(ks, ngrp, rg, tpg, tile - rg * tpg) * 64 + lane] = acc;
  }
}

// ROUNDS = loads per thread that stage the slice of x (two vectors per
// round): 2, 4 or 8 for batch <= 4, 8, 16.  SG = G / 64.  TW = tiles per
// wave.  All three are template parameters so that every load is issued
// unconditionally (clamped indices) and the compiler can count exactly the
// loads issued after each one.
template <int SG, int TW, int ROUNDS>
__global__ __launch_bounds__(64 * kKWaves) void gemv_smfmac_slice_kernel(
    int rows, int units, int sg_shift, const int32_t *__restrict__ row_ptr,
    const uint8_t *__restrict__ vals, const uint16_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *x, int batch,
    uint16_t *__restrict__ y, f4_t *__restrict__ partial) {
  typedef RowsGeom<kKUnits> Geo;  // a tile's staging area, as in the rows kernel
  constexpr int NL = Geo::kLoads, ST = Geo::kStride;
  static_assert(Geo::kRowsPerLoad == 4 && NL == 4, "a tile is 4 loads of 4 rows x 16 units");
  extern __shared__ __align__(16) uint8_t lds[];  // x: [batch][kKXStride] halfs, then [waves][Geo::kTileLds]
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int li = lane % 16, lq = lane / 16;  // the matrix layout
  const int lu = lane % 16, lr = lane / 16;  // the load layout: unit lu of row 4k + lr
  const int ksplit = gridDim.x, ngrp = gridDim.y;
  // The slices of a row group share the cache lines of its scales and
  // row_ptr: all of them run on one XCD (one L2).  Blocks go to the XCDs
  // round-robin by linear index, so linear index L takes row group
  // 8 * (L / (8 * ksplit)) + L % 8 and slice (L / 8) % ksplit; the groups
  // past the last multiple of 8 take the rest in the same way.  (Measured
  // on MI355X: 1-2 us faster than slice-major order on the 13B layers.)
  int ks, rg;
  {
    const int L = (int)(blockIdx.y * gridDim.x + blockIdx.x), ng8 = ngrp / 8 * 8;
    if (L < ng8 * ksplit) {
      rg = (L / 8) / ksplit * 8 + L % 8;
      ks = (L / 8) % ksplit;
    } else {
      const int r = L - ng8 * ksplit, rem = ngrp - ng8;  // rem >= 1 here
      rg = ng8 + r % rem;
      ks = r / rem;
    }
  }
  const int u0 = ks * kKUnits, nu = min(kKUnits, units - u0);  // live units of the slice (>= 1 by the grid)
  const int cols = units * kSegCols;
  const uint32_t nnz_row = (uint32_t)units * 32;
  const uint32_t ngroups = (uint32_t)units >> sg_shift;
  const int tile0 = (rg * kKWaves + wave) * TW;  // the wave's first tile
  uint16_t *xs = reinterpret_cast<uint16_t *>(lds);
  uint8_t *wl = lds + (size_t)batch * kKXStride * 2 + wave * Geo::kTileLds;
  u32x4_t *lv = reinterpret_cast<u32x4_t *>(wl);                                      // [16 rows][ST]
  u32x2_t *lc = reinterpret_cast<u32x2_t *>(wl + Geo::kValsBytes);                    // [16 rows][ST]
  uint16_t *lsc = reinterpret_cast<uint16_t *>(wl + Geo::kValsBytes + Geo::kCodesBytes);  // [16 / SG groups][16 rows]

  // 1. the slice of x: vector 2r + (tid / 128), 16-byte piece tid % 128 of the
  // live units (threads with a clamped index fetch, and later write, a piece
  // that another thread also writes: the same bytes to the same place)
  const int xh = threadIdx.x / 128, xp = min((int)threadIdx.x % 128, nu * 8 - 1);
  u32x4_t xg[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int v = min(2 * r + xh, batch - 1);
    xg[r] = *reinterpret_cast<const u32x4_t *>(x + (int64_t)v * cols + (int64_t)u0 * kSegCols + 8 * xp);
  }
  // x is deliberately not __restrict__: its loads then stay ordered before
  // the weight loads across the scheduling barrier (invariant loads would
  // float past it).
  __builtin_amdgcn_sched_barrier(0);

  // 2. weights: tile j of the wave, lane (unit lu, row 4k + lr).  A unit past
  // the slice's end re-reads its last live unit, and a group past it its
  // last live group; their scales are staged as +0 below, and since K % G
  // == 0 and slices start on multiples of 16 units, such units form whole
  // quantization groups, whose partial tiles (finite) are multiplied by
  // zero.  Scales: NS loads per tile, lane (row l % 16, group 4i + l / 16 of
  // the slice) -- a 64-lane load costs the address unit about the same
  // whatever its width, so the tile's 16 x 16 / SG scales take 4 / SG
  // loads, not one per load of weights (measured: the 2-byte scale and
  // 4-byte row_ptr loads, 8 per tile, cost 1.5 us of the 13824x5120 layer at
  // batch 4).  Two buffers: tile j uses buffer j % 2.
  constexpr int NG = kKUnits / SG, NS = NG / 4;  // groups per slice, scale loads per tile
  const int ngl = nu / SG;                        // live groups (nu % SG == 0: K % G == 0)
  u32x4_t wv[2][NL];
  u32x2_t wc[2][NL];
  uint16_t wsc[2][NS];
  const int ul = u0 + min(lu, nu - 1);
  auto load_tile = [&](int j, int b) {
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const uint32_t row = (uint32_t)min((tile0 + j) * 16 + 4 * k + lr, rows - 1);
      const uint32_t e0 = row * nnz_row + (uint32_t)ul * 32;
      wv[b][k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(vals + (e0 >> 1)));
      wc[b][k] = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(codes + (e0 >> 3)));
    }
    const uint32_t srow = (uint32_t)min((tile0 + j) * 16 + li, rows - 1);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int g = min(4 * i + lq, ngl - 1);
      wsc[b][i] = __builtin_nontemporal_load(scales + srow * ngroups + (uint32_t)(u0 / SG + g));
    }
  };
  // row_ptr of the wave's 16 * TW rows, one load: lane l takes row l % (16 * TW)
  const int rrow = min(tile0 * 16 + lane % (16 * TW), rows - 1);
  // 3. the slice to LDS and a block barrier (it orders LDS only) before any
  // weight load is issued.  Loads return roughly in the order the memory
  // system receives them: behind the layer's whole weight stream (every
  // wave issues its tiles at once) the slice arrived microseconds late
  // (per-wave clock stamps on a 13824x5120 layer at batch 4: median 3.4 us
  // after the wave's start, against 1.1 us when it goes first).  And a wave
  // that has issued its weight loads reaches a barrier late: with a layer's
  // loads outstanding, issue stalls until the memory system drains (median
  // 4.1 us at the barrier when it followed the weight loads).
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r)
    *reinterpret_cast<u32x4_t *>(xs + min(2 * r + xh, batch - 1) * kKXStride + 8 * xp) = xg[r];
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  load_tile(0, 0);
  if constexpr (TW > 1) load_tile(1, 1);
  const int32_t rp = row_ptr[rrow];
  __builtin_amdgcn_sched_barrier(0);

  // B lane (vector li, column quarter lq); lanes past `batch` read the last
  // real vector (their output columns are never stored)
  const uint16_t *xl = xs + min(li, batch - 1) * kKXStride + 8 * lq;
#pragma unroll
  for (int j = 0; j < TW; ++j) {
    const int b = j & 1;
    // The staging area is the wave's own, written in the load layout and
    // read back by other lanes of the wave in the matrix layout: a
    // wave-scope synchronisation before the writes of every tile after the
    // first (the previous tile's reads are done) and after the writes.
    if (j > 0) wave_lds_sync();
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      lv[(4 * k + lr) * ST + lu] = wv[b][k];
      lc[(4 * k + lr) * ST + lu] = wc[b][k];
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) lsc[(4 * i + lq) * 16 + li] = 4 * i + lq < ngl ? wsc[b][i] : (uint16_t)0;
    wave_lds_sync();
    if (j + 2 < TW) {
      __builtin_amdgcn_sched_barrier(0);
      load_tile(j + 2, b);
      __builtin_amdgcn_sched_barrier(0);
    }
    f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      // the matrix layout: lane (row li, chunk lq) takes unit 4bb + lq
      const u32x4_t v = lv[li * ST + 4 * bb + lq];
      const u32x2_t cw = lc[li * ST + 4 * bb + lq];
      uint32_t W0 = v.x, W1 = v.y, W2 = v.z, W3 = v.w, P, Q;
      transpose4(W0, W1, W2, W3);
      transpose_codes(cw.x, cw.y, P, Q);
      // the scales of the block's groups (rows 4lq..4lq+3 of each), read
      // before the matrix steps
      u32x2_t sv[4 / SG];
#pragma unroll
      for (int g = 0; g < 4 / SG; ++g)
        sv[g] = *reinterpret_cast<const u32x2_t *>(&lsc[(4 * bb / SG + g) * 16 + 4 * lq]);
      f4_t cg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // units past the slice's end read the last live unit's columns
        const int ub = min(4 * bb + s, nu - 1);
        const u32x4_t xa = *reinterpret_cast<const u32x4_t *>(xl + ub * kSegCols);
        const u32x4_t xb = *reinterpret_cast<const u32x4_t *>(xl + ub * kSegCols + 32);
        const u8_t xv = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
        const h16_t hb = __builtin_bit_cast(h16_t, xv);
        if (s == 0) cg = smfmac_step<0>(W0, hb, cg, P, Q);
        if (s == 1) cg = smfmac_step<1>(W1, hb, cg, P, Q);
        if (s == 2) cg = smfmac_step<2>(W2, hb, cg, P, Q);
        if (s == 3) cg = smfmac_step<3>(W3, hb, cg, P, Q);
        if ((s + 1) % SG == 0) {  // the group ends with this unit
          const u32x2_t g2 = sv[s / SG];
          acc[0] = fmaf(fp16_bits_to_float(g2.x & 0xFFFFu), cg[0], acc[0]);
          acc[1] = fmaf(fp16_bits_to_float(g2.x >> 16), cg[1], acc[1]);
          acc[2] = fmaf(fp16_bits_to_float(g2.y & 0xFFFFu), cg[2], acc[2]);
          acc[3] = fmaf(fp16_bits_to_float(g2.y >> 16), cg[3], acc[3]);
          cg = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
      }
    }
    slice_store(acc, tile0 + j, ks, ksplit, rg, ngrp, TW, rows, batch, y, partial);
  }

  // row_ptr check (wave-uniform).  A row stored away from the format's
  // offset is rare: the wave then recomputes its tiles' share of this slice
  // from row_ptr's offsets with a plain per-lane loop (lane (vector li,
  // quarter lq) owns rows 4lq..4lq+3 of each tile, as in the matrix
  // accumulator) and stores again, within the same tolerance.
  if (__builtin_amdgcn_ballot_w64((uint32_t)rp != (uint32_t)rrow * nnz_row) != 0) {
    const uint16_t *xv = x + (int64_t)min(li, batch - 1) * cols;
    for (int j = 0; j < TW; ++j) {
      f4_t acc;
      for (int r = 0; r < 4; ++r) {
        const int row = min((tile0 + j) * 16 + 4 * lq + r, rows - 1);
        const uint32_t rs = safe_row_start<2>(row_ptr[row], (uint32_t)(rows - 1) * nnz_row);
        float sum = 0.0f;
        for (int u = u0; u < u0 + nu; ++u) {
          float g = 0.0f;
          for (int e = 0; e < 32; ++e) {
            const uint32_t el = rs + (uint32_t)u * 32 + (uint32_t)e;
            const uint32_t word = reinterpret_cast<const uint32_t *>(vals)[el >> 3];
            const uint32_t k8 = el & 7u;
            const uint32_t slot = (k8 & 1u) ? 4u + (k8 >> 1) : (k8 >> 1);
            const int q = (int)((word >> (4 * slot)) & 0xFu) - 8;
            const uint32_t code = (codes[el >> 3] >> (2 * (el & 7u))) & 3u;
            const int col = u * kSegCols + 4 * (e / 2) + (int)code;
            g = fmaf((float)q, fp16_bits_to_float(xv[col]), g);
          }
          sum = fmaf(fp16_bits_to_float(scales[(uint32_t)row * ngroups + ((uint32_t)u >> sg_shift)]), g, sum);
        }
        acc[r] = sum;
      }
      slice_store(acc, tile0 + j, ks, ksplit, rg, ngrp, TW, rows, batch, y, partial);
    }
  }
}


// Sums the ksplit partial tiles of every row in slice order and stores y.
// One thread per (row group, tile, lane); lanes of vectors past `batch` idle.
// tpg = tiles per row group (4 or 8: bpg = tpg / 4 blocks of 256 threads per
// group).  A row group's slices ran on one XCD (the slice kernel's block
// order), and block b takes row group 8 * (b / (8 * bpg)) + b % 8 -- the
// same XCD under the round-robin placement of blocks, whose L2 may still hold
// the group's partials -- and part (b / 8) % bpg of it; the groups past the
// last multiple of 8 take the rest in the same way.
// (Measured on MI355X, 5120x13824 at batch 4 / 8 / 16: 14.23 / 14.14 / 15.96
// -> 13.90 / 13.66 / 14.59 us per call for both launches, against blocks in
// row-group order.)  The placement only affects speed: the blocks cover the
// groups exactly once under any placement.
template <int RL>
__global__ __launch_bounds__(256) void gemv_slice_reduce_kernel(
    int rows, int batch, int ngrp, int tpg, int ksplit, const f4_t *__restrict__ partial,
    uint16_t *__restrict__ y) {
  const int bpg = tpg / 4, b = (int)blockIdx.x, ng8 = ngrp / 8 * 8;
  int rgb, part;
  if (b < ng8 * bpg) {
    rgb = 8 * (b / (8 * bpg)) + b % 8;
    part = (b / 8) % bpg;
  } else {
    const int r = b - ng8 * bpg, rem = ngrp - ng8;  // rem >= 1 here
    rgb = ng8 + r % rem;
    part = r / rem;
  }
  const int gid = (rgb * bpg + part) * 256 + (int)threadIdx.x;  // < ngrp * tpg * 64
  const int lane = gid % 64, tile = (gid / 64) % tpg, rg = gid / (64 * tpg);
  const int li = lane % 16, lq = lane / 16;
  if (li >= batch) return;
  // RL (8 or 16, at least the slice count up to 16) loads in flight: every
  // slice of K <= 16384 in one round trip, summed in slice order.  (With the
  // compiler free to interleave the sums, the loads past the eighth were
  // issued only after the first had returned.)
  f4_t sum = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < ksplit; k0 += RL) {
    f4_t part[RL];
#pragma unroll
    for (int k = 0; k < RL; ++k)
      part[k] = partial[slice_tile(min(k0 + k, ksplit - 1), ngrp, rg, tpg, tile) * 64 + lane];
    __builtin_amdgcn_sched_barrier(0);  // every load issued before the first sum waits
#pragma unroll
    for (int k = 0; k < RL; ++k)
      if (k0 + k < ksplit) sum += part[k];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = (rg * tpg + tile) * 16 + 4 * lq + r;
    if (row < rows) y[(int64_t)li * rows + row] = (uint16_t)float_to_fp16_bits(sum[r]);
  }
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

// The rows kernel covers up to 8 waves of 1, 2 or 4 chunks: K <= 32768.
bool rows_kernel_fits(const i4s_packed &w) {
  const int chunks = (w.cols / kSegCols + kRUnits - 1) / kRUnits;
  return chunks <= 4 * kRMaxWaves;
}

// Shape of a rows-kernel launch: chunks per wave, waves per block, tiles
// per wave.  Two tiles per wave halve the B-fragment loads per weight byte;
// one tile per wave keeps twice the blocks for layers with few rows.
// Measured on MI355X: two tiles win from 320 tiles up (5120 rows: 7.7 / 8.0 /
// 8.8 us against 7.8 / 9.0 / 12.3 at batch 4 / 8 / 16), one tile wins at 256
// (4096 rows, 1:4: 5.2 / 5.5 / 6.7 against 6.9 / 7.1 / 7.9).
// Dynamic LDS above 64 KB needs the kernel's limit raised (once per kernel
// and device; gfx950 allows 160 KB per workgroup).  Setting it again is
// harmless, so concurrent first calls need no lock.
constexpr int kMaxDevices = 64;
template <typename Tag>
hipError_t allow_lds(const void *kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  static std::atomic<size_t> granted[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::atomic<size_t> *g = (dev >= 0 && dev < kMaxDevices) ? &granted[dev] : nullptr;
  if (g && bytes <= g->load(std::memory_order_relaxed)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && g) g->store(bytes, std::memory_order_relaxed);
  return e;
}
template <int NK, int C, int G, int T, int U, int BV> struct RowsTag {};
template <int NK, int C, int G, int T, int U, int BV> struct RowsMultiTag {};

template <int NK, int C, int G, int T, int U, int BV>
hipError_t launch_rows_t(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y, const RowsShape &r,
                         int sg_shift, hipStream_t stream) {
  const void *k = reinterpret_cast<const void *>(&gemv_smfmac_rows_kernel<NK, C, G, T, U, BV>);
  hipError_t e = allow_lds<RowsTag<NK, C, G, T, U, BV>>(k, r.lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((w.rows + 16 * T - 1) / (16 * T))), block(64 * r.waves);
  hipLaunchKernelGGL((gemv_smfmac_rows_kernel<NK, C, G, T, U, BV>), grid, block, r.lds, stream, w.rows,
                     w.cols / kSegCols, sg_shift, w.row_ptr, w.vals, w.codes, w.scales, x, batch, y);
  return hipGetLastError();
}

template <int NK, int C, int G, int T, int U, int BV>
hipError_t launch_rows_multi_t(int units, const uint16_t *x, int32_t batch, const MultiDesc &d, int blocks,
                               const RowsShape &r, hipStream_t stream) {
  const void *k = reinterpret_cast<const void *>(&gemv_smfmac_rows_multi_kernel<NK, C, G, T, U, BV>);
  hipError_t e = allow_lds<RowsMultiTag<NK, C, G, T, U, BV>>(k, r.lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemv_smfmac_rows_multi_kernel<NK, C, G, T, U, BV>), dim3((unsigned)blocks),
                     dim3(64 * r.waves), r.lds, stream, units, x, batch, d);
  return hipGetLastError();
}

// Call FN<NK, cpw, SG, tpw, U, bv>(args...) for the shape's run-time values.
// Every combination rows_shape can return is listed; anything else (and a
// group size other than 64, 128 or 256) is refused rather than run on an
// instantiation built for another shape.
#define I4S_ROWS_SG(FN, C, T, U, BV, ...)                                                \
  do {                                                                                   \
    if (sg_shift == 0) return FN<NK, C, 1, T, U, BV>(__VA_ARGS__);                       \
    if (sg_shift == 1) return FN<NK, C, 2, T, U, BV>(__VA_ARGS__);                       \
    if (sg_shift == 2) return FN<NK, C, 4, T, U, BV>(__VA_ARGS__);                       \
    return hipErrorNotSupported;                                                         \
  } while (0)
// bv 4 and 8 (1:4 only with one 8-unit chunk per wave), 16 (one tile per
// wave; four tiles of 2:4 below) or 0
#define I4S_ROWS_BV(FN, C, T, U, ...)                                                    \
  do {                                                                                   \
    if constexpr (NK != 1 || (C == 1 && U == 8)) {                                       \
      if (r.bv == 4) I4S_ROWS_SG(FN, C, T, U, 4, __VA_ARGS__);                           \
      if (r.bv == 8) I4S_ROWS_SG(FN, C, T, U, 8, __VA_ARGS__);                           \
    }                                                                                    \
    if constexpr (T == 1) {                                                              \
      if (r.bv == 16) I4S_ROWS_SG(FN, C, T, U, 16, __VA_ARGS__);                         \
    }                                                                                    \
    if (r.bv == 0) I4S_ROWS_SG(FN, C, T, U, 0, __VA_ARGS__);                             \
    return hipErrorNotSupported;                                                         \
  } while (0)
#define I4S_ROWS_DISPATCH(FN, ...)                                                       \
  do {                                                                                   \
    if (r.u == 16) {                                                                     \
      if (r.cpw == 4 && r.tpw == 1) I4S_ROWS_BV(FN, 4, 1, 16, __VA_ARGS__);             \
      if (r.cpw == 1 && r.tpw == 1) I4S_ROWS_BV(FN, 1, 1, 16, __VA_ARGS__);             \
      if (r.cpw == 1 && r.tpw == 2) I4S_ROWS_BV(FN, 1, 2, 16, __VA_ARGS__);             \
      if (r.cpw == 2 && r.tpw == 1) I4S_ROWS_BV(FN, 2, 1, 16, __VA_ARGS__);             \
      if constexpr (NK != 4) {                                                           \
        if (r.cpw == 2 && r.tpw == 2) I4S_ROWS_BV(FN, 2, 2, 16, __VA_ARGS__);           \
      }                                                                                  \
    }                                                                                    \
    if (r.u == 8 && r.cpw == 1) {                                                        \
      if (r.tpw == 1) I4S_ROWS_BV(FN, 1, 1, 8, __VA_ARGS__);                            \
      if (r.tpw == 2) I4S_ROWS_BV(FN, 1, 2, 8, __VA_ARGS__);                            \
      if constexpr (NK == 2) {                                                           \
        if (r.tpw == 4 && r.bv == 16) I4S_ROWS_SG(FN, 1, 4, 8, 16, __VA_ARGS__);       \
        if (r.tpw == 4 && r.bv == 0) I4S_ROWS_SG(FN, 1, 4, 8, 0, __VA_ARGS__);         \
      }                                                                                  \
    }                                                                                    \
    return hipErrorNotSupported;                                                         \
  } while (0)

template <int NK>
hipError_t launch_rows(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                       hipStream_t stream) {
  const RowsShape r = rows_shape(w.cols / kSegCols, (w.rows + 15) / 16, batch, NK);
  const int sg_shift = w.group_size == 64 ? 0 : (w.group_size == 128 ? 1 : 2);
  I4S_ROWS_DISPATCH(launch_rows_t, w, x, batch, y, r, sg_shift, stream);
}

template <int NK>
hipError_t launch_rows_multi(const i4s_packed *w, int32_t n, const uint16_t *x, int32_t batch,
                             uint16_t *const *y, hipStream_t stream) {
  const int units = w[0].cols / kSegCols;
  // The chunk width decides how a row's sum is split across waves, and so
  // its rounding: fuse only layers whose single calls take the same width,
  // and keep it (the tile count per wave does not change any result bit).
  const int u0 = rows_shape(units, (w[0].rows + 15) / 16, batch, NK).u;
  int total_tiles = 0;
  for (int m = 0; m < n; ++m) {
    if (rows_shape(units, (w[m].rows + 15) / 16, batch, NK).u != u0) return hipErrorNotSupported;
    total_tiles += (w[m].rows + 15) / 16;
  }
  const RowsShape r = rows_shape(units, total_tiles, batch, NK, u0);
  const int sg_shift = w[0].group_size == 64 ? 0 : (w[0].group_size == 128 ? 1 : 2);
  MultiDesc d = {};
  d.n = n;
  int blocks = 0;
  for (int m = 0; m < n; ++m) {
    blocks += (w[m].rows + 16 * r.tpw - 1) / (16 * r.tpw);
    d.block_end[m] = blocks;
    d.rows[m] = w[m].rows;
    d.sg_shift[m] = sg_shift;
    d.row_ptr[m] = w[m].row_ptr;
    d.vals[m] = w[m].vals;
    d.codes[m] = w[m].codes;
    d.scales[m] = w[m].scales;
    d.y[m] = y[m];
  }
  I4S_ROWS_DISPATCH(launch_rows_multi_t, units, x, batch, d, blocks, r, stream);
}
#undef I4S_ROWS_DISPATCH
#undef I4S_ROWS_SG

hipError_t launch_smfmac(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                         hipStream_t stream) {
  if (rows_kernel_fits(w)) return launch_rows<2>(w, x, batch, y, stream);
  const dim3 grid((unsigned)((w.rows + 15) / 16)), block(64 * kMWaves);
  if (w.group_size == 64)
    hipLaunchKernelGGL(gemv_smfmac_kernel<1>, grid, block, 0, stream, w.rows, w.cols, w.row_ptr, w.vals,
                       w.codes, w.scales, x, batch, y);
  else if (w.group_size == 128)
    hipLaunchKernelGGL(gemv_smfmac_kernel<2>, grid, block, 0, stream, w.rows, w.cols, w.row_ptr, w.vals,
                       w.codes, w.scales, x, batch, y);
  else
    hipLaunchKernelGGL(gemv_smfmac_kernel<4>, grid, block, 0, stream, w.rows, w.cols, w.row_ptr, w.vals,
                       w.codes, w.scales, x, batch, y);
  return hipGetLastError();
}

template <int SG, int TW, int RN>
hipError_t launch_slice_t(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                          const SplitPlan &pl, f4_t *partial, hipStream_t stream) {
  const size_t lds = (size_t)batch * kKXStride * 2 + kKWaves * RowsGeom<kKUnits>::kTileLds;  // <= 61,952 bytes
  const int sg_shift = SG == 1 ? 0 : (SG == 2 ? 1 : 2);
  hipLaunchKernelGGL((gemv_smfmac_slice_kernel<SG, TW, RN>), dim3((unsigned)pl.ksplit, (unsigned)pl.row_groups),
                     dim3(64 * kKWaves), lds, stream, w.rows, w.cols / kSegCols, sg_shift, w.row_ptr, w.vals,
                     w.codes, w.scales, x, batch, y, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.ksplit == 1) return e;
  const int tpg = kKWaves * TW;
  const unsigned threads = (unsigned)pl.row_groups * (unsigned)tpg * 64u;  // a multiple of 256
  if (pl.ksplit <= 8)
    hipLaunchKernelGGL(gemv_slice_reduce_kernel<8>, dim3(threads / 256), dim3(256), 0, stream, w.rows, batch,
                       pl.row_groups, tpg, pl.ksplit, partial, y);
  else
    hipLaunchKernelGGL(gemv_slice_reduce_kernel<16>, dim3(threads / 256), dim3(256), 0, stream, w.rows, batch,
                       pl.row_groups, tpg, pl.ksplit, partial, y);
  return hipGetLastError();
}

template <int SG, int TW>
hipError_t launch_slice_tw(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                           const SplitPlan &pl, f4_t *partial, hipStream_t stream) {
  if (batch <= 4) return launch_slice_t<SG, TW, 2>(w, x, batch, y, pl, partial, stream);
  if (batch <= 8) return launch_slice_t<SG, TW, 4>(w, x, batch, y, pl, partial, stream);
  return launch_slice_t<SG, TW, 8>(w, x, batch, y, pl, partial, stream);
}

template <int SG>
hipError_t launch_slice_sg(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                           const SplitPlan &pl, f4_t *partial, hipStream_t stream) {
  if (pl.tw == 1) return launch_slice_tw<SG, 1>(w, x, batch, y, pl, partial, stream);
  if (pl.tw == 2) return launch_slice_tw<SG, 2>(w, x, batch, y, pl, partial, stream);
  return hipErrorNotSupported;
}

hipError_t launch_smfmac_slice(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                               const SplitPlan &pl, void *workspace, hipStream_t stream) {
  f4_t *partial = static_cast<f4_t *>(workspace);
  switch (w.group_size) {
    case 64: return launch_slice_sg<1>(w, x, batch, y, pl, partial, stream);
    case 128: return launch_slice_sg<2>(w, x, batch, y, pl, partial, stream);
    case 256: return launch_slice_sg<4>(w, x, batch, y, pl, partial, stream);
    default: return hipErrorNotSupported;
  }
}

template <int NK>
hipError_t launch_nk(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                     hipStream_t stream) {
  if (batch == 2) {
    const hipError_t e = launch_gemv_bv(w, x, batch, y, stream);
    if (e != hipErrorNotSupported) return e;
  }
  if (NK == 2 && batch >= I4S_MATRIX_CORE_MIN_BATCH) {
    return launch_smfmac(w, x, batch, y, stream);
  }
  if ((NK == 1 || NK == 4) && batch >= I4S_MATRIX_CORE_MIN_BATCH && rows_kernel_fits(w)) {
    return launch_rows<NK>(w, x, batch, y, stream);
  }
  if (batch <= 1) {
    return launch_gemv_b1(w, x, y, stream);
  }
  if (batch <= 2) return launch_t<NK, 2, 4>(w, x, batch, y, stream);
  if (batch <= 4) return launch_t<NK, 4, 2>(w, x, batch, y, stream);
  if (batch <= 8) return launch_t<NK, 8, 2>(w, x, batch, y, stream);
  return launch_t<NK, 16, 1>(w, x, batch, y, stream);
}

}  // namespace

hipError_t launch_gemv_ws(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                          const SplitPlan &pl, void *workspace, hipStream_t stream) {
  if (pl.ksplit >= 1) return launch_smfmac_slice(w, x, batch, y, pl, workspace, stream);
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

hipError_t launch_gemv_multi(const i4s_packed *w, int32_t n, const uint16_t *x, int32_t batch,
                             uint16_t *const *y, hipStream_t stream) {
  bool same = true;  // one pattern, one group size, one K
  // a layer that a single call runs on the batch-2 VALU kernel keeps that
  // kernel, so that fused results stay those of single calls bit for bit
  bool valu_b2 = gemv_bv_applies(w[0], batch);
  for (int m = 1; m < n; ++m) {
    same &= w[m].n_keep == w[0].n_keep && w[m].group_size == w[0].group_size && w[m].cols == w[0].cols;
    valu_b2 |= gemv_bv_applies(w[m], batch);
  }
  if (n > 1 && same) {
    if (batch == 1) {
      const hipError_t e = launch_gemv_b1_multi(w, n, x, y, stream);
      if (e != hipErrorNotSupported) return e;
    } else if (!valu_b2 && batch >= I4S_MATRIX_CORE_MIN_BATCH && rows_kernel_fits(w[0])) {
      const hipError_t e = w[0].n_keep == 2   ? launch_rows_multi<2>(w, n, x, batch, y, stream)
                           : w[0].n_keep == 1 ? launch_rows_multi<1>(w, n, x, batch, y, stream)
                                              : launch_rows_multi<4>(w, n, x, batch, y, stream);
      if (e != hipErrorNotSupported) return e;
    }
  }
  for (int m = 0; m < n; ++m) {
    const hipError_t e = launch_gemv(w[m], x, batch, y[m], stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace i4s
