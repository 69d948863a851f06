// Batch-2 SparseGEMV kernel for gfx950: y = W_hat x for two activation
// vectors over the 2-bit CSR INT4 format, on the VALU.
//
// Method: "Efficient LLM-based Advertising via Model Compression and Parallel
// Verification", section 3.3, "Computational Acceleration" (INT4 weights
// widened to fp16 with bit operations, 2-bit indices selecting activations),
// with the small verification batches of its section 3.4 in view.
//
// The batch-1 kernel's mapping (8-wave blocks, one row per wave, lane l owns
// 64-column units l and l + 64, every load issued before the first wait) with
// both vectors' activations staged in LDS.  Each unit's weights are decoded
// once -- dequantized fp16 pairs and, for 2:4 and 1:4, the v_perm_b32
// selectors -- and then multiplied with each vector in turn, so the second
// vector costs one selection and one v_dot2 per group.  Used for batch 2 on
// layers of at most 8192 rows and K <= 4096; taller or wider layers and larger
// batches go to the sparse matrix cores.

#include "i4s_gemv_common.h"

namespace i4s {
namespace {

// The 64 activations of unit u of one staged vector (eight 16-byte reads).
__device__ inline void lds_unit_x2(const uint16_t *xs, int u, uint32_t (&xr)[32]) {
  const uint4 *xv = reinterpret_cast<const uint4 *>(xs + __umul24((uint32_t)u, kStrideB1));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 t = xv[i];
    xr[4 * i] = t.x; xr[4 * i + 1] = t.y; xr[4 * i + 2] = t.z; xr[4 * i + 3] = t.w;
  }
}

// The decoded form of one unit: NP exact fp16 weight pairs and, for 2:4 and
// 1:4, the v_perm_b32 selectors that pick each pair's activations.
template <int NK>
struct UnitDecoded {
  static constexpr int NP = 8 * NK;            // weight pairs per unit
  static constexpr int NS = NK == 4 ? 1 : (NK == 2 ? 16 : 16);  // selector words
  h2_t q[NP];
  uint32_t sel[NS];
};

template <int NK>
__device__ inline void unit_decode(const UnitRegs<NK> &u, const uint32_t *lut, UnitDecoded<NK> &d) {
#pragma unroll
  for (int j = 0; j < 2 * NK; ++j) dequant_word(u.v[j], &d.q[4 * j]);
  if constexpr (NK == 2) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t me = (u.c[c] << 2) & 0x3C3C3C3Cu;
      uint32_t mo = (u.c[c] >> 2) & 0x3C3C3C3Cu;
      opaque(me);
      opaque(mo);
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) {
        const uint32_t m = (gi & 1) ? mo : me;
        d.sel[8 * c + gi] = lut_read(lut, (m >> (8 * (gi >> 1))) & 0xFFu);
      }
    }
  } else if constexpr (NK == 1) {
    uint32_t me = (u.c[0] << 3) & 0x78787878u;
    uint32_t mo = (u.c[0] >> 1) & 0x78787878u;
    opaque(me);
    opaque(mo);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t m = (k & 1) ? mo : me;
      const u32x2_lut_t sp = lut_read2(lut, (m >> (8 * (k >> 1))) & 0xFFu);
      d.sel[2 * k] = sp.x;
      d.sel[2 * k + 1] = sp.y;
    }
  }
}

// sum_e q_e * x_(column of e) over the unit, for one vector's activations
template <int NK>
__device__ inline float unit_dot_decoded(const UnitDecoded<NK> &d, const uint32_t (&xr)[32]) {
  float g = 0.0f;
  if constexpr (NK == 2) {
#pragma unroll
    for (int grp = 0; grp < 16; ++grp) {
      const uint32_t xp = __builtin_amdgcn_perm(xr[2 * grp + 1], xr[2 * grp], d.sel[grp]);
      g = __builtin_amdgcn_fdot2(d.q[grp], as_h2(xp), g, false);
    }
  } else if constexpr (NK == 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t xa = __builtin_amdgcn_perm(xr[4 * k + 1], xr[4 * k], d.sel[2 * k]);
      const uint32_t xb = __builtin_amdgcn_perm(xr[4 * k + 3], xr[4 * k + 2], d.sel[2 * k + 1]);
      g = __builtin_amdgcn_fdot2(d.q[k], as_h2(xa | xb), g, false);
    }
  } else {
#pragma unroll
    for (int p = 0; p < 32; ++p) g = __builtin_amdgcn_fdot2(d.q[p], as_h2(xr[p]), g, false);
  }
  return g;
}

// BV vectors (batch <= BV; vectors past the batch re-read the last one and
// are not stored), one row per wave, 8 waves per block, UPL units per lane.
// LDS: x as [BV][units][kStrideB1] halfs.  shape = units | sg_shift << 16.
template <int NK, int BV, int UPL>
__global__ __launch_bounds__(512) void gemv_bv_direct_kernel(
    int rows, int shape, const int32_t *__restrict__ row_ptr, const uint8_t *__restrict__ vals,
    const uint16_t *__restrict__ codes, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    int batch, uint16_t *__restrict__ y) {
  extern __shared__ __align__(16) uint16_t xs[];
  __shared__ __align__(8) uint32_t lut[32];
  constexpr int WAVES = 8;
  const int units = shape & 0xFFFF, sg_shift = shape >> 16;
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const int row = blockIdx.x * WAVES + wave;
  const int nvec = units * (kSegCols / 8);  // 16-byte pieces of one vector
  const uint32_t nnz_row = (uint32_t)units * 16 * NK;
  const uint32_t ngroups = (uint32_t)units >> sg_shift;
  const uint32_t xstride = (uint32_t)units * kStrideB1;  // halfs per vector in LDS

  // 1. activations of all BV vectors (BV * nvec <= BV * 512 * UPL pieces)
  constexpr int XP = BV * UPL;
  u32x4_t xg[XP];
  uint32_t xo[XP];
#pragma unroll
  for (int j = 0; j < XP; ++j) {
    const int piece = min((int)threadIdx.x + j * 64 * WAVES, BV * nvec - 1);
    const int v = piece / nvec, i = piece - v * nvec;
    xo[j] = __umul24((uint32_t)v, xstride) + __umul24((uint32_t)i >> 3, kStrideB1) + 8u * ((uint32_t)i & 7u);
    const uint32_t src = (uint32_t)min(v, batch - 1) * (uint32_t)nvec + (uint32_t)i;
    xg[j] = *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const char *>(x) + 16u * src);
  }
  issue_fence();

  // 2. weights (rows past the end re-read the last row, never stored)
  const bool rvalid = row < rows;
  const int rr = min(row, rows - 1);
  const uint32_t rstart = (uint32_t)rr * nnz_row, srow = (uint32_t)rr * ngroups;
  UnitRegs<NK> wr[UPL];
#pragma unroll
  for (int k = 0; k < UPL; ++k) {
    const int u = min(lane + 64 * k, units - 1);
    load_unit_nt<NK>(wr[k], vals, codes, scales, rstart + (uint32_t)u * 16 * NK, srow + ((uint32_t)u >> sg_shift));
    issue_fence();
  }
  const int32_t rp = row_ptr[min((int)(blockIdx.x * WAVES + threadIdx.x / 64), rows - 1)];
  __builtin_amdgcn_sched_barrier(0);

  // 3. stage x
#pragma unroll
  for (int j = 0; j < XP; ++j) *reinterpret_cast<u32x4_t *>(xs + xo[j]) = xg[j];
  init_tables<NK>(lut);
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // 4. decode each unit once, then one dot product per vector
  float acc[BV];
#pragma unroll
  for (int v = 0; v < BV; ++v) acc[v] = 0.0f;
  auto pass = [&](const UnitRegs<NK> (&w)[UPL]) {
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
      const int u = lane + 64 * k;
      const int uc = min(u, units - 1);
      UnitDecoded<NK> d;
      unit_decode<NK>(w[k], lut, d);
      const float sc = fp16_bits_to_float(w[k].s);
#pragma unroll
      for (int v = 0; v < BV; ++v) {
        uint32_t xr[32];
        lds_unit_x2(xs + v * xstride, uc, xr);
        const float a = fmaf(sc, unit_dot_decoded<NK>(d, xr), acc[v]);
        acc[v] = u < units ? a : acc[v];
      }
    }
  };
  pass(wr);
  __builtin_amdgcn_sched_barrier(0);
  // row_ptr check after the decode (wave-uniform): a row stored elsewhere is
  // fetched again into registers of its own and recomputed
  if ((uint32_t)rp != rstart) {
#pragma unroll
    for (int v = 0; v < BV; ++v) acc[v] = 0.0f;
    UnitRegs<NK> w2[UPL];
    const uint32_t rs = safe_row_start<NK>(rp, (uint32_t)(rows - 1) * nnz_row);
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
      const int u = min(lane + 64 * k, units - 1);
      load_unit<NK>(w2[k], vals, codes, scales, rs + (uint32_t)u * 16 * NK, srow + ((uint32_t)u >> sg_shift));
    }
    pass(w2);
  }

  // 5. reduce and store
#pragma unroll
  for (int v = 0; v < BV; ++v) {
    const float t = wave_sum(acc[v]);
    if (lane == 0 && rvalid && v < batch) y[(int64_t)v * rows + row] = (uint16_t)float_to_fp16_bits(t);
  }
}

// ---------------------------------------------------------------------------
// dispatch

template <int NK, int BV, int UPL>
hipError_t launch_bv_t(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y, hipStream_t stream) {
  const int units = w.cols / kSegCols;
  const size_t lds = (size_t)BV * units * kStrideB1 * 2;
  const int sg_shift = w.group_size == 64 ? 0 : (w.group_size == 128 ? 1 : 2);
  const dim3 grid((unsigned)((w.rows + 7) / 8)), block(512);
  hipLaunchKernelGGL((gemv_bv_direct_kernel<NK, BV, UPL>), grid, block, lds, stream, w.rows,
                     units | (sg_shift << 16), w.row_ptr, w.vals, w.codes, w.scales, x, batch, y);
  return hipGetLastError();
}

template <int NK, int BV>
hipError_t launch_bv_u(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y, hipStream_t stream) {
  switch ((w.cols / kSegCols + 63) / 64) {
    case 1: return launch_bv_t<NK, BV, 1>(w, x, batch, y, stream);
    default: return launch_bv_t<NK, BV, 2>(w, x, batch, y, stream);
  }
}

}  // namespace

// Measured on MI355X (cold, us per call, this kernel against the matrix-core
// kernel at batch 2): 4096x4096 2:4 4.04 / 4.45 and 1:4 3.51 / 4.43, but
// 5120x5120 2:4 7.05 / 6.65 and 13824x5120 2:4 19.3 / 11.3 (every block
// stages both vectors, and tall layers have many blocks); at batch 3 and 4
// the matrix cores win everywhere (5120x5120 b4: 13.3 against 6.9).  So:
// batch 2, at most I4S_BATCH2_VALU_MAX_ROWS rows and I4S_BATCH2_VALU_MAX_K
// columns (8192 and 4096).
bool gemv_bv_applies(const i4s_packed &w, int32_t batch) {
  return batch == 2 && w.rows <= I4S_BATCH2_VALU_MAX_ROWS && w.cols <= I4S_BATCH2_VALU_MAX_K;
}

hipError_t launch_gemv_bv(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y, hipStream_t stream) {
  if (!gemv_bv_applies(w, batch)) return hipErrorNotSupported;
  switch (w.n_keep) {
    case 1: return launch_bv_u<1, 2>(w, x, batch, y, stream);
    case 2: return launch_bv_u<2, 2>(w, x, batch, y, stream);
    default: return launch_bv_u<4, 2>(w, x, batch, y, stream);
  }
}

}  // namespace i4s
