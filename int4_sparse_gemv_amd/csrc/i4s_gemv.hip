// SparseGEMV kernels for gfx950: y = W_hat x over the 2-bit CSR INT4 format.
//
// Method: "Efficient LLM-based Advertising via Model Compression and Parallel
// Verification", section 3.3, "Computational Acceleration": activations are
// staged in on-chip shared memory (LDS here) by the whole block, INT4 weights
// are widened to fp16 with a few bit operations, and the 2-bit indices packed
// in uint16 words are decoded with shifts and masks.  The design below is
// written for CDNA4 (wave64, v_perm_b32, v_dot2_f32_f16, 64 KB+ LDS), not
// taken from the page's NVIDIA kernel.
//
// Mapping.  A block is 4 waves; each wave owns RPW consecutive rows.  A row
// is cut into 64-column "units" (16 groups of 4 columns: 8*NK bytes of vals,
// 4*NK bytes of codes, one scale); lane l takes units l, l+64, ...  Adjacent
// lanes therefore read adjacent 16-byte pieces of a row (dwordx4 for 2:4),
// and one unit never straddles a quantization group.  The RPW rows of a wave
// share the same columns, so each activation fetch from LDS feeds RPW rows.
//
// Per 8 stored elements (one 32-bit vals word) the decode is one shift, four
// v_and_or_b32 that drop nibble pairs into the mantissa of 1024.0 (fp16
// 0x6400) and four packed fp16 adds/fmas that remove the bias exactly; the
// nibble interleave of the format puts elements (2p, 2p+1) in bits 4p and
// 16+4p so one mask yields one pair.  For 2:4, a group's 4-bit code builds a
// v_perm_b32 selector that picks the two kept activations out of the group's
// four, and v_dot2_f32_f16 multiplies and accumulates in fp32.  The group
// scale is applied once per unit.
//
// Batch: BT activation vectors (BT >= batch, rounded up to 1, 2, 4, 8, 16;
// the extra vectors are zero in LDS and never stored).  When BT*K*2 bytes do
// not fit the LDS budget the K axis is processed in chunks, re-staging x.

#include "i4s_internal.h"

namespace i4s {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsBudget = 64 * 1024;  // bytes of LDS for staged activations

__device__ inline h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

// Four exact fp16 pairs (q_{2p}, q_{2p+1}), p = 0..3, of one vals word.
__device__ inline void dequant_word(uint32_t w, h2_t q[4]) {
  const uint32_t magic = 0x64006400u;  // 1024.0 in both halves
  const uint32_t t = w >> 8;
  const h2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2_t bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  // slots 0/4 and 2/6: nibble in mantissa bits 0..3 -> 1024 + u
  q[0] = as_h2((w & 0x000F000Fu) | magic) + bias;
  q[2] = as_h2((t & 0x000F000Fu) | magic) + bias;
  // slots 1/5 and 3/7: nibble in mantissa bits 4..7 -> 1024 + 16u
  q[1] = __builtin_elementwise_fma(as_h2((w & 0x00F000F0u) | magic), sixteenth, bias16);
  q[3] = __builtin_elementwise_fma(as_h2((t & 0x00F000F0u) | magic), sixteenth, bias16);
}

// v_perm_b32 selector taking fp16 lanes cf and cs of a group's four
// activations (held as two dwords {x0|x1<<16, x2|x3<<16}) into (lo, hi):
// bytes [2cf, 2cf+1, 2cs, 2cs+1].  h = cf | cs << 2.  The multiply spreads
// the two 2-bit fields into four byte lanes without carries between them.
__device__ inline uint32_t pair_selector(uint32_t h) {
  return ((h * 0x808202u) & 0x06060606u) | 0x01000100u;
}

__device__ inline float fp16_bits_to_float(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// float -> fp16 bits, round to nearest even
__device__ inline uint32_t float_to_fp16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int NK>
struct UnitRegs {
  uint32_t v[2 * NK];                 // vals words of the unit
  uint32_t c[NK < 4 ? NK : 1];        // code dwords (16 codes each)
  uint32_t s;                         // scale bits
};

template <int NK>
__device__ inline void load_unit(UnitRegs<NK> &r, const uint8_t *__restrict__ vals,
                                 const uint16_t *__restrict__ codes,
                                 const uint16_t *__restrict__ scales, int64_t elem0,
                                 int64_t scale_idx) {
  const uint32_t *vp = reinterpret_cast<const uint32_t *>(vals + elem0 / 2);
  if constexpr (NK == 1) {
    const uint2 a = *reinterpret_cast<const uint2 *>(vp);
    r.v[0] = a.x; r.v[1] = a.y;
  } else if constexpr (NK == 2) {
    const uint4 a = *reinterpret_cast<const uint4 *>(vp);
    r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
  } else {
    const uint4 a = reinterpret_cast<const uint4 *>(vp)[0];
    const uint4 b = reinterpret_cast<const uint4 *>(vp)[1];
    r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
    r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
  }
  if constexpr (NK == 1) {
    r.c[0] = *reinterpret_cast<const uint32_t *>(codes + elem0 / 8);
  } else if constexpr (NK == 2) {
    const uint2 c = *reinterpret_cast<const uint2 *>(codes + elem0 / 8);
    r.c[0] = c.x; r.c[1] = c.y;
  }
  r.s = scales[scale_idx];
}

template <int NK>
__device__ inline void zero_unit(UnitRegs<NK> &r) {
#pragma unroll
  for (int i = 0; i < 2 * NK; ++i) r.v[i] = 0x88888888u;  // q = 0
#pragma unroll
  for (int i = 0; i < (NK < 4 ? NK : 1); ++i) r.c[i] = 0x44444444u;  // valid codes
  r.s = 0u;
}

// Accumulate one unit of RPW rows into acc[r][b].  xs points at the LDS copy
// of the unit's 64 columns for batch vector 0; vector b is xstride halfs on.
template <int NK, int BT, int RPW>
__device__ inline void compute_unit(const UnitRegs<NK> (&u)[RPW], const uint16_t *xs, int xstride,
                                    float (&acc)[RPW][BT]) {
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
          const uint32_t sel = pair_selector((cw >> (4 * p)) & 0xFu);
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
      uint4 xg[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) xg[b] = *reinterpret_cast<const uint4 *>(xs + b * xstride + 8 * j);
#pragma unroll
      for (int r = 0; r < RPW; ++r)
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          g[r][b] = __builtin_amdgcn_fdot2(q[r][0], as_h2(xg[b].x), g[r][b], false);
          g[r][b] = __builtin_amdgcn_fdot2(q[r][1], as_h2(xg[b].y), g[r][b], false);
          g[r][b] = __builtin_amdgcn_fdot2(q[r][2], as_h2(xg[b].z), g[r][b], false);
          g[r][b] = __builtin_amdgcn_fdot2(q[r][3], as_h2(xg[b].w), g[r][b], false);
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
    uint16_t *__restrict__ y, int kc_cols) {
  extern __shared__ uint16_t xs[];  // [BT][kc_cols]
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int row0 = (blockIdx.x * kWaves + wave) * RPW;
  const int sg = group_size / kSegCols;  // units per quantization group
  const int ngroups = cols / group_size;

  // Row starts come from row_ptr (CSR); every row holds cols*NK/4 elements.
  int64_t rstart[RPW];
  bool rvalid[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    rvalid[r] = row0 + r < rows;
    rstart[r] = rvalid[r] ? (int64_t)row_ptr[row0 + r] : 0;
  }

  float acc[RPW][BT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[r][b] = 0.0f;

  for (int k0 = 0; k0 < cols; k0 += kc_cols) {
    const int kcn = min(kc_cols, cols - k0);
    const int ub = k0 / kSegCols, ue = (k0 + kcn) / kSegCols;

    // issue the first weight loads of this chunk before staging x
    int u = ub + lane;
    bool has = u < ue;
    UnitRegs<NK> cur[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if (has && rvalid[r])
        load_unit<NK>(cur[r], vals, codes, scales, rstart[r] + (int64_t)u * 16 * NK,
                      (int64_t)(row0 + r) * ngroups + u / sg);
      else
        zero_unit<NK>(cur[r]);
    }

    if (k0 > 0) __syncthreads();  // previous chunk fully consumed
    {
      const int vec_per_row = kcn / 8;  // uint4 = 8 halfs
      const int total = BT * vec_per_row;
      for (int i = threadIdx.x; i < total; i += kThreads) {
        const int b = i / vec_per_row, c = i % vec_per_row;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (b < batch) v = *reinterpret_cast<const uint4 *>(x + (int64_t)b * cols + k0 + 8 * c);
        *reinterpret_cast<uint4 *>(xs + b * kc_cols + 8 * c) = v;
      }
    }
    __syncthreads();

    while (has) {
      const int un = u + 64;
      const bool hn = un < ue;
      UnitRegs<NK> nxt[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        if (hn && rvalid[r])
          load_unit<NK>(nxt[r], vals, codes, scales, rstart[r] + (int64_t)un * 16 * NK,
                        (int64_t)(row0 + r) * ngroups + un / sg);
        else
          zero_unit<NK>(nxt[r]);
      }
      compute_unit<NK, BT, RPW>(cur, xs + (u - ub) * kSegCols, kc_cols, acc);
#pragma unroll
      for (int r = 0; r < RPW; ++r) cur[r] = nxt[r];
      u = un;
      has = hn;
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

template <int NK, int BT, int RPW>
hipError_t launch_t(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                    hipStream_t stream) {
  int kc = (kLdsBudget / (BT * 2)) / kSegCols * kSegCols;
  if (kc > w.cols) kc = w.cols;
  const size_t lds = (size_t)BT * kc * 2;
  const int rows_per_block = kWaves * RPW;
  const dim3 grid((unsigned)((w.rows + rows_per_block - 1) / rows_per_block)), block(kThreads);
  hipLaunchKernelGGL((gemv_kernel<NK, BT, RPW>), grid, block, lds, stream, w.rows, w.cols,
                     w.group_size, w.row_ptr, w.vals, w.codes, w.scales, x, batch, y, kc);
  return hipGetLastError();
}

template <int NK>
hipError_t launch_nk(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                     hipStream_t stream) {
  if (batch <= 1) return launch_t<NK, 1, 4>(w, x, batch, y, stream);
  if (batch <= 2) return launch_t<NK, 2, 4>(w, x, batch, y, stream);
  if (batch <= 4) return launch_t<NK, 4, 2>(w, x, batch, y, stream);
  if (batch <= 8) return launch_t<NK, 8, 2>(w, x, batch, y, stream);
  return launch_t<NK, 16, 1>(w, x, batch, y, stream);
}

}  // namespace

hipError_t launch_gemv(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                       hipStream_t stream) {
  switch (w.n_keep) {
    case 1: return launch_nk<1>(w, x, batch, y, stream);
    case 2: return launch_nk<2>(w, x, batch, y, stream);
    default: return launch_nk<4>(w, x, batch, y, stream);
  }
}

}  // namespace i4s
