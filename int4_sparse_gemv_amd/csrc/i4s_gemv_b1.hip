// Batch-1 SparseGEMV kernels for gfx950: y = W_hat x over the 2-bit CSR INT4
// format, one activation vector.
//
// Method: "Efficient LLM-based Advertising via Model Compression and Parallel
// Verification", section 3.3, "Computational Acceleration": the activation
// vector is staged in on-chip shared memory (LDS here) by the whole block,
// INT4 weights are widened to fp16 in registers and the 2-bit indices pick
// the activations each kept weight multiplies.  No matrix instructions: at
// batch 1 the work is a stream of packed bytes with a few VALU operations
// per element.
//
// Mapping.  A block is 8 waves; each wave owns RPW consecutive rows.  A row
// is cut into 64-column "units" (16 groups of 4 columns: 8*NK bytes of vals,
// 4*NK bytes of codes, one scale); lane l takes units l, l+64, ...  Adjacent
// lanes therefore read adjacent 16-byte pieces of a row (dwordx4 for 2:4),
// and one unit never straddles a quantization group.  The RPW rows of a wave
// share the same columns, so each activation fetch from LDS feeds RPW rows.
// For 2:4 and 1:4 v_perm_b32 picks the activations: with one row per wave
// the 2:4 selectors are computed from the code nibbles (a multiply and a
// mask), otherwise they come from a 16-entry table in LDS.  v_dot2_f32_f16
// multiplies and accumulates in fp32; the group scale is applied once per
// unit.
//
// Row starts: the kernels read row_ptr, but issue the weight loads of a row
// at the offset the format prescribes (row * K * N / 4) without waiting for
// that read; when row_ptr disagrees, the row is fetched again from row_ptr's
// offset.  A dependent round trip to memory is thus kept off the common path.
//
// LDS layout of x: each 64-column unit occupies 72 halfs, so the 16-byte
// reads that 64 lanes issue for 64 different units fall in distinct banks.

#include "i4s_gemv_common.h"

namespace i4s {
namespace {

// ---------------------------------------------------------------------------
// batch-1 kernel (any N): the lane's 64 activations live in registers

template <int NK>
__device__ inline float unit_dot_b1(const UnitRegs<NK> &u, const uint32_t (&xr)[32], const uint32_t *lut) {
  float g = 0.0f;
  if constexpr (NK == 2) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {  // code dword c: groups 8c..8c+7
      uint32_t me = (u.c[c] << 2) & 0x3C3C3C3Cu;  // byte k: 4 * code nibble of group 8c+2k
      uint32_t mo = (u.c[c] >> 2) & 0x3C3C3C3Cu;  // byte k: 4 * code nibble of group 8c+2k+1
      opaque(me);
      opaque(mo);
#pragma unroll
      for (int half = 0; half < 2; ++half) {  // vals word j = 2c + half: groups 8c+4half .. +3
        h2_t q[4];
        dequant_word(u.v[2 * c + half], q);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int gi = 4 * half + p;  // group within the code dword
          const uint32_t m = (gi & 1) ? mo : me;
          const uint32_t sel = lut_read(lut, (m >> (8 * (gi >> 1))) & 0xFFu);
          const int grp = 8 * c + gi;
          const uint32_t xp = __builtin_amdgcn_perm(xr[2 * grp + 1], xr[2 * grp], sel);
          g = __builtin_amdgcn_fdot2(q[p], as_h2(xp), g, false);
        }
      }
    }
  } else if constexpr (NK == 1) {
    // one code dword per unit: nibble k holds the codes of elements 2k, 2k+1
    const uint32_t me = (u.c[0] << 3) & 0x78787878u;  // byte b: 8 * nibble 2b
    const uint32_t mo = (u.c[0] >> 1) & 0x78787878u;  // byte b: 8 * nibble 2b+1
#pragma unroll
    for (int j = 0; j < 2; ++j) {  // vals word j: elements (= groups) 8j..8j+7
      h2_t q[4];
      dequant_word(u.v[j], q);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int k = 4 * j + p;  // pair k: groups 2k, 2k+1
        const uint32_t m = (k & 1) ? mo : me;
        const u32x2_lut_t sel = lut_read2(lut, (m >> (8 * (k >> 1))) & 0xFFu);
        const uint32_t xa = __builtin_amdgcn_perm(xr[4 * k + 1], xr[4 * k], sel.x);
        const uint32_t xb = __builtin_amdgcn_perm(xr[4 * k + 3], xr[4 * k + 2], sel.y);
        g = __builtin_amdgcn_fdot2(q[p], as_h2(xa | xb), g, false);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // vals word j: columns 8j..8j+7
      h2_t q[4];
      dequant_word(u.v[j], q);
#pragma unroll
      for (int p = 0; p < 4; ++p) g = __builtin_amdgcn_fdot2(q[p], as_h2(xr[4 * j + p]), g, false);
    }
  }
  return g;
}

// unit_dot_b1 in two steps, for 2:4 and 1:4: the activations each kept
// weight multiplies (they depend on the codes and x only, so they can be
// picked while the unit's vals are still on their way), then the products
// (the same dot2 operations in the same order: the same bits).
template <int NK>
constexpr int kPicked = NK == 2 ? 16 : 8;  // activation pairs per unit
template <int NK>
__device__ inline void unit_pick_b1(const UnitRegs<NK> &u, const uint32_t (&xr)[32], const uint32_t *lut,
                                    uint32_t (&xp)[kPicked<NK>]) {
  if constexpr (NK == 2) {
    // The selectors are computed rather than read from the table here: byte
    // k of me / mo is the code nibble of group 2k / 2k+1, and the selector is
    // pair_selector's multiply and masks -- a v_mul_u32_u24 that reads the
    // nibble's byte straight from the register, then one v_and_or_b32.  Two
    // VALU per group against one plus an LDS read (measured on the 4096x4096
    // and 4096x11008 2:4 layers: 3.32 -> 3.28 and 6.10 -> 5.94 us; the
    // two-row decode below keeps the table, where the computed form was
    // slower).
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      uint32_t me = u.c[c] & 0x0F0F0F0Fu;
      uint32_t mo = (u.c[c] >> 4) & 0x0F0F0F0Fu;
      opaque(me);
      opaque(mo);
#pragma unroll
      for (int gi = 0; gi < 8; ++gi) {
        const uint32_t m = (gi & 1) ? mo : me;
        const uint32_t sel = and_or(((m >> (8 * (gi >> 1))) & 0xFFu) * 0x808202u, 0x06060606u, 0x01000100u);
        const int grp = 8 * c + gi;
        xp[grp] = __builtin_amdgcn_perm(xr[2 * grp + 1], xr[2 * grp], sel);
      }
    }
  } else {
    const uint32_t me = (u.c[0] << 3) & 0x78787878u;
    const uint32_t mo = (u.c[0] >> 1) & 0x78787878u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t m = (k & 1) ? mo : me;
      const u32x2_lut_t sel = lut_read2(lut, (m >> (8 * (k >> 1))) & 0xFFu);
      xp[k] = __builtin_amdgcn_perm(xr[4 * k + 1], xr[4 * k], sel.x) |
              __builtin_amdgcn_perm(xr[4 * k + 3], xr[4 * k + 2], sel.y);
    }
  }
}
template <int NK>
__device__ inline float unit_products_b1(const UnitRegs<NK> &u, const uint32_t (&xp)[kPicked<NK>]) {
  float g = 0.0f;
#pragma unroll
  for (int j = 0; j < kPicked<NK> / 4; ++j) {  // vals word j: activation pairs 4j..4j+3
    h2_t q[4];
    dequant_word(u.v[j], q);
#pragma unroll
    for (int p = 0; p < 4; ++p) g = __builtin_amdgcn_fdot2(q[p], as_h2(xp[4 * j + p]), g, false);
  }
  return g;
}

// The 64 activations of unit u from the block's LDS copy (eight 16-byte reads).
__device__ inline void lds_unit_x(const uint16_t *xs, int u, uint32_t (&xr)[32]) {
  const uint4 *xv = reinterpret_cast<const uint4 *>(xs + __umul24((uint32_t)u, kStrideB1));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 t = xv[i];
    xr[4 * i] = t.x; xr[4 * i + 1] = t.y; xr[4 * i + 2] = t.z; xr[4 * i + 3] = t.w;
  }
}

// Dense INT4 in the one-launch batch-1 kernel: the offsets are removed once
// per unit instead of once per element.  The nibbles enter v_dot2 as the raw
// magic-number halves, 1024 + u for the low nibble of each byte and
// 1024 + 16u for the high one (elements 2, 3, 6, 7 of every 8), and the
// block stages the activations of those columns divided by 16 (exact for
// normal values), so each product is (1024 + u) x or (64 + u) x.  The unit's
// offset term, D = 1032 * sum(x, low columns) + 1152 * sum(x / 16, high
// columns), is subtracted after the unit's dot products: sum((u - 8) x).  D
// is summed while x is staged: a 16-byte piece's share with four v_dot2
// (1032 and 1152 are exact in fp16), the unit's eight pieces -- eight
// consecutive lanes -- with three DPP additions (quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror).  The sums are of terms ~1000x larger
// than the result, in fp32: the error stays ~1e-4 of the tolerance's
// sum |w x|.  32 fewer VALU per unit-row than the exact per-element form.
__device__ inline void dense_stage_piece(u32x4_t &v, float *dsum, int xi_raw, int nvec) {
  const h2_t s16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  v.y = __builtin_bit_cast(uint32_t, as_h2(v.y) * s16);  // columns 2, 3 of the piece
  v.w = __builtin_bit_cast(uint32_t, as_h2(v.w) * s16);  // columns 6, 7
  const h2_t klo = {(_Float16)1032.0f, (_Float16)1032.0f}, khi = {(_Float16)1152.0f, (_Float16)1152.0f};
  float p = __builtin_amdgcn_fdot2(as_h2(v.x), klo, 0.0f, false);
  p = __builtin_amdgcn_fdot2(as_h2(v.y), khi, p, false);
  p = __builtin_amdgcn_fdot2(as_h2(v.z), klo, p, false);
  p = __builtin_amdgcn_fdot2(as_h2(v.w), khi, p, false);
  p = dpp_rot_add<0xB1>(p);
  p = dpp_rot_add<0x4E>(p);
  p = dpp_rot_add<0x141>(p);
  if ((xi_raw & 7) == 0 && xi_raw < nvec) dsum[xi_raw >> 3] = p;
}

__device__ inline float unit_dot_dense_raw(const UnitRegs<4> &u, const uint32_t (&xr)[32], float d) {
  const uint32_t magic = 0x64006400u;
  float g = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {  // vals word j: columns 8j..8j+7
    const uint32_t w = u.v[j], t = w >> 8;
    g = __builtin_amdgcn_fdot2(as_h2(and_or(w, 0x000F000Fu, magic)), as_h2(xr[4 * j]), g, false);
    g = __builtin_amdgcn_fdot2(as_h2(and_or(w, 0x00F000F0u, magic)), as_h2(xr[4 * j + 1]), g, false);
    g = __builtin_amdgcn_fdot2(as_h2(and_or(t, 0x000F000Fu, magic)), as_h2(xr[4 * j + 2]), g, false);
    g = __builtin_amdgcn_fdot2(as_h2(and_or(t, 0x00F000F0u, magic)), as_h2(xr[4 * j + 3]), g, false);
  }
  return g - d;
}

template <int NK, int RPW, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_b1_kernel(
    int rows, int cols, int group_size, const int32_t *__restrict__ row_ptr,
    const uint8_t *__restrict__ vals, const uint16_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, int kc_units) {
  extern __shared__ __align__(16) uint16_t xs[];  // [kc_units][kStrideB1]
  __shared__ __align__(8) uint32_t lut[32];
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int row0 = (blockIdx.x * WAVES + wave) * RPW;
  const int units = cols / kSegCols;
  const uint32_t nnz_row = (uint32_t)cols / 4 * NK;
  const int sg_shift = group_size == 64 ? 0 : (group_size == 128 ? 1 : 2);  // log2(G / 64)
  const uint32_t ngroups = (uint32_t)(cols / group_size);

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

  float acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;

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
      const int nvec = (ue - ub) * (kSegCols / 8);  // uint4 = 8 halfs
      for (int i = threadIdx.x; i < nvec; i += 64 * WAVES) {
        const int un = i >> 3, part = i & 7;
        *reinterpret_cast<uint4 *>(xs + un * kStrideB1 + 8 * part) =
            *reinterpret_cast<const uint4 *>(x + (int64_t)ub * kSegCols + 8 * i);
      }
      if (ub == 0) init_tables<NK>(lut);
    }
    __syncthreads();

    if (ub == 0) {
      // row_ptr check (wave-uniform): re-fetch rows stored elsewhere
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
      // the end keep the body one basic block, so the compiler cannot hoist
      // one iteration's LDS reads into the previous one.
      const int uc = hn ? un : ue - 1;
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        load_unit<NK>(nxt[r], vals, codes, scales, rstart[r] + (uint32_t)uc * 16 * NK,
                      srow[r] + ((uint32_t)uc >> sg_shift));
      uint32_t xr[32];
      const uint4 *xv = reinterpret_cast<const uint4 *>(xs + (u - ub) * kStrideB1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 t = xv[i];
        xr[4 * i] = t.x; xr[4 * i + 1] = t.y; xr[4 * i + 2] = t.z; xr[4 * i + 3] = t.w;
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const float gsum = unit_dot_b1<NK>(cur[r], xr, lut);
        acc[r] = fmaf(fp16_bits_to_float(cur[r].s), gsum, acc[r]);
      }
#pragma unroll
      for (int r = 0; r < RPW; ++r) cur[r] = nxt[r];
      u = un;
      has = hn;
    }
  }

#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float t = wave_sum(acc[r]);
    if (lane == 0 && rvalid[r]) y[row0 + r] = (uint16_t)float_to_fp16_bits(t);
  }
}

// ---------------------------------------------------------------------------
// batch-1 kernel for rows of at most 64 * UPL units: every load up front.
//
// A wave issues the block's share of the activation loads first, then all of
// its lanes' weight loads (UPL units per lane, nontemporal: the weights are
// read once).  Vector loads retire in issue order, so the LDS write of x --
// and the block barrier after it -- waits for the activations only, not for
// the weight stream; each wave starts computing as soon as its own weights
// are in, which overlaps the decode with the stream.

// units = K / 64; sg_shift = log2(G / 64).  Shapes arrive pre-divided so the
// prologue before the first load is a handful of scalar shifts.  `blk` is
// the block's index within its layer; xs and lut are the block's LDS.
template <int NK, int RPW, int UPL, int WAVES>
__device__ __forceinline__ void b1_direct_body(
    int blk, int rows, int units, int sg_shift, const int32_t *__restrict__ row_ptr,
    const uint8_t *__restrict__ vals, const uint16_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y, uint16_t *xs, uint32_t *lut) {
  const int lane = threadIdx.x % 64;
  // The wave index is uniform: row offsets are then scalar arithmetic, and
  // the weight loads take a scalar base plus a 32-bit per-lane offset.
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const int row0 = (blk * WAVES + wave) * RPW;
  const int nvec = units * (kSegCols / 8);  // uint4 pieces of x
  const uint32_t nnz_row = (uint32_t)units * 16 * NK;
  const uint32_t ngroups = (uint32_t)units >> sg_shift;

  // 1. activations (nvec <= 512 * UPL, so XP pieces per thread cover them).
  // Every load below is unconditional, at a clamped index, so the wait before
  // the LDS write counts exactly the loads issued after it.
  constexpr int XP = (8 * UPL + WAVES - 1) / WAVES;
  u32x4_t xg[XP];  // a vector type: a plain load, not an aggregate copy the optimizer may re-place
  uint32_t xi[XP];
#pragma unroll
  for (int j = 0; j < XP; ++j) {
    xi[j] = (uint32_t)min((int)threadIdx.x + j * 64 * WAVES, nvec - 1);
    xg[j] = *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const char *>(x) + 16u * xi[j]);
  }
  issue_fence();

  // 2. weights: rows past the end re-read the last row (never stored)
  uint32_t rstart[RPW], srow[RPW];
  bool rvalid[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    rvalid[r] = row0 + r < rows;
    const int rr = min(row0 + r, rows - 1);
    rstart[r] = (uint32_t)rr * nnz_row;
    srow[r] = (uint32_t)rr * ngroups;
  }
  // In the order the decode consumes them: unit by unit, the rows of a unit
  // together.  With one row per wave (2:4 and 1:4), every unit's codes go
  // first: the activations a unit's weights multiply are then picked while
  // its vals are still streaming in, and what is left after the last vals
  // arrive is the dequantization and the dot products.  (Per-wave clock
  // stamps on a 4096x4096 2:4 layer: the decode after the weights' arrival
  // took 0.56 us at the median, the last 0.7 us of the launch.)
  constexpr bool kCodesFirst = RPW == 1 && NK != 4;
  UnitRegs<NK> wr[UPL][RPW];
  if constexpr (kCodesFirst) {
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
      const int u = min(lane + 64 * k, units - 1);  // lanes past the row re-read its last unit
      load_codes_nt<NK>(wr[k][0], codes, rstart[0] + (uint32_t)u * 16 * NK);
    }
    issue_fence();
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
      const int u = min(lane + 64 * k, units - 1);
      load_vals_scale_nt<NK>(wr[k][0], vals, scales, rstart[0] + (uint32_t)u * 16 * NK,
                             srow[0] + ((uint32_t)u >> sg_shift));
      issue_fence();
    }
  } else {
#pragma unroll
    for (int k = 0; k < UPL; ++k) {
      const int u = min(lane + 64 * k, units - 1);  // lanes past the row re-read its last unit
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        load_unit_nt<NK>(wr[k][r], vals, codes, scales, rstart[r] + (uint32_t)u * 16 * NK,
                         srow[r] + ((uint32_t)u >> sg_shift));
      issue_fence();
    }
  }
  // row_ptr: a vector load, issued last and needed only after decoding.  (A
  // scalar load would share its counter with LDS and, returning out of
  // order, hold up the block barrier and the first LDS reads.)
  // (The index is formed from the per-lane wave number so that it stays a
  // vector load.)
  const int row0_v = (blk * WAVES + (int)threadIdx.x / 64) * RPW;
  int32_t rp[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) rp[r] = row_ptr[min(row0_v + r, rows - 1)];
  __builtin_amdgcn_sched_barrier(0);

  // 3. stage x in LDS (threads with a clamped index write the same piece
  // to the same place again)
  // dense: the per-unit offset terms follow the activations in LDS
  float *dsum = reinterpret_cast<float *>(xs + units * kStrideB1);
#pragma unroll
  for (int j = 0; j < XP; ++j) {
    u32x4_t v = xg[j];
    if constexpr (NK == 4) dense_stage_piece(v, dsum, (int)threadIdx.x + j * 64 * WAVES, nvec);
    *reinterpret_cast<u32x4_t *>(xs + __umul24(xi[j] >> 3, kStrideB1) + 8 * (xi[j] & 7)) = v;
  }
  init_tables<NK>(lut);
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // one unit-row's dot product (u: the unit whose activations xr holds)
  auto dot_unit = [&](const UnitRegs<NK> &t, const uint32_t (&xr)[32], int u) -> float {
    if constexpr (NK == 4) return unit_dot_dense_raw(t, xr, dsum[u]);
    else return unit_dot_b1<NK>(t, xr, lut);
  };

  // 4. decode and accumulate.  The activations of the lane's first unit are
  // read from LDS before the first wait for weights, so those reads overlap
  // the stream; each unit's activations then feed all RPW rows.
  uint32_t xr0[32];
  lds_unit_x(xs, min(lane, units - 1), xr0);
  __builtin_amdgcn_sched_barrier(0);
  float acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;
  // One row per wave: lanes past the row's end compute on its last unit and
  // discard the result (a select, not a branch: behind a branch the compiler
  // moved the dense weight loads down into the decode block, after the
  // barrier).  Two or more rows keep the branch: without it their register
  // count rose from ~75 to ~120, too many for three blocks per CU.
  uint32_t xp[kCodesFirst ? kPicked<NK> : 1];
  if constexpr (kCodesFirst) {
    unit_pick_b1<NK>(wr[0][0], xr0, lut, xp);  // waits for the codes only
    __builtin_amdgcn_sched_barrier(0);          // every pick before the first wait for vals
  }
#pragma unroll
  for (int k = 0; k < UPL; ++k) {
    const int u = lane + 64 * k;
    if constexpr (kCodesFirst) {
      const float a = fmaf(fp16_bits_to_float(wr[k][0].s), unit_products_b1<NK>(wr[k][0], xp), acc[0]);
      acc[0] = u < units ? a : acc[0];
      if (k + 1 < UPL) {  // the next unit's picks, while its vals arrive
        uint32_t xr[32];
        lds_unit_x(xs, min(u + 64, units - 1), xr);
        unit_pick_b1<NK>(wr[k + 1][0], xr, lut, xp);
      }
    } else if constexpr (RPW == 1) {
      uint32_t xr[32];
      if (k == 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i) xr[i] = xr0[i];
      } else {
        lds_unit_x(xs, min(u, units - 1), xr);
      }
      const float a = fmaf(fp16_bits_to_float(wr[k][0].s), dot_unit(wr[k][0], xr, min(u, units - 1)), acc[0]);
      acc[0] = u < units ? a : acc[0];
    } else {
      auto decode = [&]() {
        uint32_t xr[32];
        if (k == 0) {
#pragma unroll
          for (int i = 0; i < 32; ++i) xr[i] = xr0[i];
        } else {
          lds_unit_x(xs, u, xr);
        }
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
          const float gsum = dot_unit(wr[k][r], xr, u);
          acc[r] = fmaf(fp16_bits_to_float(wr[k][r].s), gsum, acc[r]);
        }
      };
      // a wave-uniform test first: the loads then have uses in two blocks
      // and stay where they were issued
      if (64 * (k + 1) <= units) decode();
      else if (u < units) decode();
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // The row_ptr check comes after the decode, so the common case never waits
  // for row_ptr; a row stored away from the format's offset (wave-uniform) is
  // fetched from row_ptr's offset into registers of its own and decoded again.
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    if ((uint32_t)rp[r] != rstart[r]) {
      acc[r] = 0.0f;
#pragma unroll
      for (int k = 0; k < UPL; ++k) {
        const int u = min(lane + 64 * k, units - 1);
        UnitRegs<NK> t;
        load_unit<NK>(t, vals, codes, scales,
                      safe_row_start<NK>(rp[r], (uint32_t)(rows - 1) * nnz_row) + (uint32_t)u * 16 * NK,
                      srow[r] + ((uint32_t)u >> sg_shift));
        if (lane + 64 * k < units) {
          uint32_t xr[32];
          lds_unit_x(xs, u, xr);
          acc[r] = fmaf(fp16_bits_to_float(t.s), dot_unit(t, xr, u), acc[r]);
        }
      }
    }
  }

  // 5. reduce and store
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float t = wave_sum(acc[r]);
    if (lane == 0 && rvalid[r]) y[row0 + r] = (uint16_t)float_to_fp16_bits(t);
  }
}

template <int NK, int RPW, int UPL, int WAVES>
// shape = units | sg_shift << 16: with the two sizes in one dword the
// arguments fit the 14 preloaded SGPRs, y included, so no wave loads an
// argument from memory (the store of y used to wait for one).
__global__ __launch_bounds__(64 * WAVES) void gemv_b1_direct_kernel(
    int rows, int shape, const int32_t *__restrict__ row_ptr,
    const uint8_t *__restrict__ vals, const uint16_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ y) {
  extern __shared__ __align__(16) uint16_t xs[];  // [units][kStrideB1]
  __shared__ __align__(8) uint32_t lut[32];
  b1_direct_body<NK, RPW, UPL, WAVES>(blockIdx.x, rows, shape & 0xFFFF, shape >> 16, row_ptr, vals, codes, scales,
                                      x, y, xs, lut);
}

// Several layers that share x in one launch (horizontal fusion): each block
// finds its layer from the cumulative block counts (a few scalar compares on
// preloaded arguments) and runs the single-layer body on it.
template <int NK, int RPW, int UPL, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_b1_direct_multi_kernel(
    int units, const uint16_t *__restrict__ x, MultiDesc d) {
  extern __shared__ __align__(16) uint16_t xs[];  // [units][kStrideB1]
  __shared__ __align__(8) uint32_t lut[32];
  int m = 0;
#pragma unroll
  for (int i = 1; i < kMaxMulti; ++i) m += (i < d.n && (int)blockIdx.x >= d.block_end[i - 1]) ? 1 : 0;
  const int first = m == 0 ? 0 : d.block_end[m - 1];
  b1_direct_body<NK, RPW, UPL, WAVES>((int)blockIdx.x - first, d.rows[m], units, d.sg_shift[m], d.row_ptr[m],
                                      d.vals[m], d.codes[m], d.scales[m], x, d.y[m], xs, lut);
}

// ---------------------------------------------------------------------------
// dispatch

// Batch-1 kernel: 8 waves per block (512 threads), RPW rows per wave.
constexpr int kB1Waves = 8;

template <int NK, int RPW, int UPL>
hipError_t launch_b1_direct(const i4s_packed &w, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const int units = w.cols / kSegCols;
  const size_t lds = (size_t)units * kStrideB1 * 2 + (NK == 4 ? (size_t)units * 4 : 0);  // + dense offset terms
  const int rows_per_block = kB1Waves * RPW;
  const dim3 grid((unsigned)((w.rows + rows_per_block - 1) / rows_per_block)), block(64 * kB1Waves);
  const int sg_shift = w.group_size == 64 ? 0 : (w.group_size == 128 ? 1 : 2);
  hipLaunchKernelGGL((gemv_b1_direct_kernel<NK, RPW, UPL, kB1Waves>), grid, block, lds, stream, w.rows,
                     units | (sg_shift << 16), w.row_ptr, w.vals, w.codes, w.scales, x, y);
  return hipGetLastError();
}

template <int NK, int RPW, int UPL>
hipError_t launch_b1_direct_multi(const i4s_packed *w, int32_t n, const uint16_t *x, uint16_t *const *y,
                                  hipStream_t stream) {
  const int units = w[0].cols / kSegCols;
  const size_t lds = (size_t)units * kStrideB1 * 2 + (NK == 4 ? (size_t)units * 4 : 0);  // + dense offset terms
  const int rows_per_block = kB1Waves * RPW;
  MultiDesc d = {};
  d.n = n;
  int blocks = 0;
  for (int m = 0; m < n; ++m) {
    blocks += (w[m].rows + rows_per_block - 1) / rows_per_block;
    d.block_end[m] = blocks;
    d.rows[m] = w[m].rows;
    d.sg_shift[m] = w[m].group_size == 64 ? 0 : (w[m].group_size == 128 ? 1 : 2);
    d.row_ptr[m] = w[m].row_ptr;
    d.vals[m] = w[m].vals;
    d.codes[m] = w[m].codes;
    d.scales[m] = w[m].scales;
    d.y[m] = y[m];
  }
  hipLaunchKernelGGL((gemv_b1_direct_multi_kernel<NK, RPW, UPL, kB1Waves>), dim3((unsigned)blocks),
                     dim3(64 * kB1Waves), lds, stream, units, x, d);
  return hipGetLastError();
}

template <int NK, int RPW>
hipError_t launch_b1_multi_t(const i4s_packed *w, int32_t n, const uint16_t *x, uint16_t *const *y,
                             hipStream_t stream) {
  switch ((w[0].cols / kSegCols + 63) / 64) {
    case 1: return launch_b1_direct_multi<NK, RPW, 1>(w, n, x, y, stream);
    case 2: return launch_b1_direct_multi<NK, RPW, 2>(w, n, x, y, stream);
    case 3: return launch_b1_direct_multi<NK, RPW, 3>(w, n, x, y, stream);
    default: return launch_b1_direct_multi<NK, RPW, 4>(w, n, x, y, stream);
  }
}

template <int NK, int RPW>
hipError_t launch_b1(const i4s_packed &w, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const int units = w.cols / kSegCols;
  switch ((units + 63) / 64) {
    case 1: return launch_b1_direct<NK, RPW, 1>(w, x, y, stream);
    case 2: return launch_b1_direct<NK, RPW, 2>(w, x, y, stream);
    case 3: return launch_b1_direct<NK, RPW, 3>(w, x, y, stream);
    case 4: return launch_b1_direct<NK, RPW, 4>(w, x, y, stream);
    default: break;  // longer rows: the pipelined kernel
  }
  int kc = kLdsBudget / (kStrideB1 * 2);
  if (kc > units) kc = units;
  const size_t lds = (size_t)kc * kStrideB1 * 2;
  const int rows_per_block = kB1Waves * RPW;
  const dim3 grid((unsigned)((w.rows + rows_per_block - 1) / rows_per_block)), block(64 * kB1Waves);
  hipLaunchKernelGGL((gemv_b1_kernel<NK, RPW, kB1Waves>), grid, block, lds, stream, w.rows, w.cols,
                     w.group_size, w.row_ptr, w.vals, w.codes, w.scales, x, y, kc);
  return hipGetLastError();
}

// Rows per wave of the batch-1 kernel.  One row per wave keeps 2+ blocks on
// every CU up to ~8k rows; taller matrices take two rows per wave so each
// block's staged activations feed more rows.
int b1_rows_per_wave(int rows) { return rows > 8192 ? 2 : 1; }

}  // namespace

hipError_t launch_gemv_b1(const i4s_packed &w, const uint16_t *x, uint16_t *y, hipStream_t stream) {
  const bool two = b1_rows_per_wave(w.rows) == 2;
  switch (w.n_keep) {
    case 1: return two ? launch_b1<1, 2>(w, x, y, stream) : launch_b1<1, 1>(w, x, y, stream);
    case 2: return two ? launch_b1<2, 2>(w, x, y, stream) : launch_b1<2, 1>(w, x, y, stream);
    default: return two ? launch_b1<4, 2>(w, x, y, stream) : launch_b1<4, 1>(w, x, y, stream);
  }
}

hipError_t launch_gemv_b1_multi(const i4s_packed *w, int32_t n, const uint16_t *x, uint16_t *const *y,
                                hipStream_t stream) {
  const int units = w[0].cols / kSegCols;
  if (units > 256) return hipErrorNotSupported;
  int max_rows = 0;
  for (int m = 0; m < n; ++m) {
    if (w[m].n_keep != w[0].n_keep || w[m].cols != w[0].cols) return hipErrorNotSupported;
    max_rows = max_rows > w[m].rows ? max_rows : w[m].rows;
  }
  // rows per wave as for the tallest layer alone
  const int rpw = b1_rows_per_wave(max_rows);
  switch (w[0].n_keep) {
    case 1: return rpw == 2 ? launch_b1_multi_t<1, 2>(w, n, x, y, stream) : launch_b1_multi_t<1, 1>(w, n, x, y, stream);
    case 2: return rpw == 2 ? launch_b1_multi_t<2, 2>(w, n, x, y, stream) : launch_b1_multi_t<2, 1>(w, n, x, y, stream);
    default: return rpw == 2 ? launch_b1_multi_t<4, 2>(w, n, x, y, stream) : launch_b1_multi_t<4, 1>(w, n, x, y, stream);
  }
}

}  // namespace i4s
