// Packer kernels for gfx950: N:4 pruning by magnitude or by the full
// importance score, symmetric INT4 group quantization with fp16 scales, the
// exact-SSE choice of the group size, and the encoding of the 2-bit CSR
// buffers.
//
// Method: "Efficient LLM-based Advertising via Model Compression and Parallel
// Verification", section 3.2 (N:M pruning ordered by the Eq. (3) importance
// |W_ij| * ||X_j||_2 + |W_ij| * |dE/dW_ij|, which orders by |w| when the
// activation norm is constant and the gradient term is absent; layer-adaptive
// group-wise INT4 quantization) and section 3.3
// ("Sparse Index Structure": CSR with 2-bit in-group column indices packed
// into uint16 words from the least significant bits).
//
// Work decomposition: one thread per (row, 64-column segment).  A segment
// holds 16 groups of 4 columns and never straddles a quantization group, so
// the amax of a group of G columns is the max over G/64 neighbouring
// segments; those sit in neighbouring lanes of one wave (K is a multiple of
// G), and a lane shuffle combines them.
//
// Importance: with caller-supplied column norms n_j (fp32) and/or gradients
// g_ij (fp16) the score is |w| * (n_j + |g_ij|) in fp32, the sum and the
// product each rounded to nearest even (n_j = 1 and g_ij = 0 when absent).
// The scores are non-negative (or -0 / +inf), so their bit patterns with the
// sign cleared order like their values.
//
// Exactness: every fp16 value is an integer multiple of 2^-24, and so is an
// fp16 scale times a small integer; the squared errors are therefore summed
// as exact unsigned 128-bit integers (units of 2^-48).  The scale is
// fp16_rne(amax / 7): the fp32 quotient is correctly rounded, and since the
// binary expansion of m/7 repeats with a 3-bit period that is never 000 or
// 111, that intermediate rounding cannot land on or cross an fp16 rounding
// boundary.  q rounds a correctly rounded fp32 w / s half-to-even: a
// quotient that is not exactly k + 1/2 lies at least 2^-11 (relative) away
// from it, far beyond fp32's error.

#include "i4s_internal.h"

namespace i4s {
namespace {

struct U128 {
  uint64_t lo, hi;
};

__device__ inline void add128(U128 &a, uint64_t lo, uint64_t hi) {
  const uint64_t s = a.lo + lo;
  a.hi += hi + (s < lo ? 1ull : 0ull);
  a.lo = s;
}

__device__ inline U128 wave_sum128(U128 v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t lo = __shfl_xor(v.lo, off, 64);
    const uint64_t hi = __shfl_xor(v.hi, off, 64);
    add128(v, lo, hi);
  }
  return v;
}

// Value of an fp16 bit pattern in units of 2^-24 (exact).
__device__ inline int64_t fp16_units(uint32_t b) {
  const uint32_t e = (b >> 10) & 0x1Fu;
  const uint32_t m = b & 0x3FFu;
  const int64_t v = e == 0 ? (int64_t)m : ((int64_t)(m | 0x400u) << (e - 1));
  return (b & 0x8000u) ? -v : v;
}

__device__ inline float fp16_bits_to_float(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// float -> fp16 bits, round to nearest even
__device__ inline uint32_t float_to_fp16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// fp16 bits of round_to_nearest_even(amax / 7); amax is a 15-bit magnitude.
__device__ inline uint32_t scale_bits(uint32_t amax_mag) {
  const float a = fp16_bits_to_float(amax_mag);
  const float s = a / 7.0f;  // correctly rounded (built with the IEEE divide)
  return float_to_fp16_bits(s);
}

// q = clamp(rne(w / s), -8, 7); 0 when s == 0.
__device__ inline int quantize(uint32_t w_bits, uint32_t s_bits) {
  if ((s_bits & 0x7FFFu) == 0) return 0;
  const float r = fp16_bits_to_float(w_bits) / fp16_bits_to_float(s_bits);
  float q = rintf(r);
  q = fminf(fmaxf(q, -8.0f), 7.0f);
  return (int)q;
}

// In-group columns kept for one group of 4, ascending.  The kept set is the
// NK largest keys; among equal keys the lower column wins.
template <int NK>
__device__ inline void select_group(const uint32_t key[4], int code[NK]) {
  const uint32_t m0 = key[0], m1 = key[1], m2 = key[2], m3 = key[3];
  if constexpr (NK == 4) {
    code[0] = 0; code[1] = 1; code[2] = 2; code[3] = 3;
  } else {
    // rank = number of elements that beat this one
    const int r0 = (m1 > m0) + (m2 > m0) + (m3 > m0);
    const int r1 = (m0 >= m1) + (m2 > m1) + (m3 > m1);
    const int r2 = (m0 >= m2) + (m1 >= m2) + (m3 > m2);
    if constexpr (NK == 2) {
      const bool k0 = r0 < 2, k1 = r1 < 2, k2 = r2 < 2;
      const int r3 = (m0 >= m3) + (m1 >= m3) + (m2 >= m3);
      const bool k3 = r3 < 2;
      code[0] = k0 ? 0 : (k1 ? 1 : 2);
      code[1] = k3 ? 3 : (k2 ? 2 : 1);
    } else {
      code[0] = r0 == 0 ? 0 : (r1 == 0 ? 1 : (r2 == 0 ? 2 : 3));
    }
  }
}

__device__ inline uint32_t pick4(const uint32_t h[4], int c) {
  return c == 0 ? h[0] : (c == 1 ? h[1] : (c == 2 ? h[2] : h[3]));
}

// Optional inputs of the importance score (device pointers, may be null).
struct ImportanceIn {
  const float *norm;     // [cols] fp32 column norms
  const uint16_t *grad;  // [rows][cols] fp16 gradient bits
};

constexpr uint32_t kFlagNonfiniteWeight = kPackFlagNonfiniteWeight;
constexpr uint32_t kFlagBadNorm = kPackFlagBadNorm, kFlagBadGrad = kPackFlagBadGrad;

// Load the 64 fp16 values of a segment as 64 bit patterns (zero if !valid)
// and compute the kept elements (bits) and codes.  HN / HG: column norms /
// gradients are given.  Returns the flag bits this segment raises.
template <int NK, bool HN, bool HG>
__device__ inline uint32_t load_and_select(const uint16_t *__restrict__ w, ImportanceIn imp,
                                           int64_t row, int seg, int cols, bool valid,
                                           uint32_t kv[16 * NK], int kc[16 * NK]) {
  uint32_t words[32], gwords[HG ? 32 : 1];
  float nv[HN ? 64 : 1];
  const int64_t off = row * (int64_t)cols + (int64_t)seg * kSegCols;
  if (valid) {
    const uint4 *src = reinterpret_cast<const uint4 *>(w + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = src[i];
      words[4 * i + 0] = v.x; words[4 * i + 1] = v.y;
      words[4 * i + 2] = v.z; words[4 * i + 3] = v.w;
    }
    if constexpr (HG) {
      const uint4 *gsrc = reinterpret_cast<const uint4 *>(imp.grad + off);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 v = gsrc[i];
        gwords[4 * i + 0] = v.x; gwords[4 * i + 1] = v.y;
        gwords[4 * i + 2] = v.z; gwords[4 * i + 3] = v.w;
      }
    }
    if constexpr (HN) {
      const float4 *nsrc = reinterpret_cast<const float4 *>(imp.norm + (int64_t)seg * kSegCols);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 v = nsrc[i];
        nv[4 * i + 0] = v.x; nv[4 * i + 1] = v.y;
        nv[4 * i + 2] = v.z; nv[4 * i + 3] = v.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) words[i] = 0u;
    if constexpr (HG) {
#pragma unroll
      for (int i = 0; i < 32; ++i) gwords[i] = 0u;
    }
    if constexpr (HN) {
#pragma unroll
      for (int i = 0; i < 64; ++i) nv[i] = 0.0f;
    }
  }
  uint32_t flags = 0;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    uint32_t h[4];
    h[0] = words[2 * t] & 0xFFFFu;
    h[1] = words[2 * t] >> 16;
    h[2] = words[2 * t + 1] & 0xFFFFu;
    h[3] = words[2 * t + 1] >> 16;
    uint32_t key[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if ((h[c] & 0x7C00u) == 0x7C00u) flags |= kFlagNonfiniteWeight;
      if constexpr (!HN && !HG) {
        key[c] = h[c] & 0x7FFFu;  // finite fp16 magnitudes order like their low 15 bits
      } else {
        float n = 1.0f, g = 0.0f;
        if constexpr (HN) {
          n = nv[4 * t + c];
          const uint32_t nb = __builtin_bit_cast(uint32_t, n);
          // finite and not below zero (-0 is allowed)
          if ((nb & 0x7F800000u) == 0x7F800000u || (nb > 0x80000000u)) flags |= kFlagBadNorm;
        }
        if constexpr (HG) {
          const uint32_t gb = (gwords[2 * t + (c >> 1)] >> (16 * (c & 1))) & 0xFFFFu;
          if ((gb & 0x7C00u) == 0x7C00u) flags |= kFlagBadGrad;
          g = fp16_bits_to_float(gb & 0x7FFFu);
        }
        const float a = n + g;  // one rounding; -0 + +0 = +0
        const float sc = fp16_bits_to_float(h[c] & 0x7FFFu) * a;
        key[c] = __builtin_bit_cast(uint32_t, sc) & 0x7FFFFFFFu;
      }
    }
    int code[NK];
    select_group<NK>(key, code);
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      kc[NK * t + k] = code[k];
      kv[NK * t + k] = pick4(h, code[k]);
    }
  }
  return flags;
}

template <int NK>
__device__ inline uint32_t segment_amax(const uint32_t kv[16 * NK]) {
  uint32_t a = 0;
#pragma unroll
  for (int e = 0; e < 16 * NK; ++e) a = max(a, kv[e] & 0x7FFFu);
  return a;
}

// Combine the amax of the G/64 neighbouring segments of one group.
__device__ inline uint32_t group_amax(uint32_t a, int group_size) {
  if (group_size >= 128) a = max(a, (uint32_t)__shfl_xor((int)a, 1, 64));
  if (group_size >= 256) a = max(a, (uint32_t)__shfl_xor((int)a, 2, 64));
  return a;
}

template <int NK, bool HN, bool HG>
__global__ __launch_bounds__(kPackThreads) void pack_analyze_kernel(
    const uint16_t *__restrict__ w, ImportanceIn imp, int rows, int cols, int adaptive,
    uint8_t *__restrict__ ws) {
  const int S = cols / kSegCols;
  const int64_t total = (int64_t)rows * S;
  const int64_t f = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
  const bool valid = f < total;
  const int64_t row = valid ? f / S : 0;
  const int seg = valid ? (int)(f % S) : 0;

  uint32_t kv[16 * NK];
  int kc[16 * NK];
  const uint32_t flags = load_and_select<NK, HN, HG>(w, imp, row, seg, cols, valid, kv, kc);
  if (flags) atomicOr(reinterpret_cast<unsigned int *>(ws + kWsFlagOffset), flags);
  if (!adaptive) return;  // uniform across the grid

  const uint32_t a64 = segment_amax<NK>(kv);
  U128 part[3];
#pragma unroll
  for (int ci = 0; ci < 3; ++ci) {
    const int G = 64 << ci;
    const uint32_t s = scale_bits(group_amax(a64, G));
    const int64_t s_units = fp16_units(s);
    U128 acc = {0ull, 0ull};
#pragma unroll
    for (int e = 0; e < 16 * NK; ++e) {
      const int q = quantize(kv[e], s);
      const int64_t n = fp16_units(kv[e]) - s_units * q;
      const uint64_t a = (uint64_t)(n < 0 ? -n : n);
      add128(acc, a * a, __umul64hi(a, a));
    }
    part[ci] = wave_sum128(acc);
  }

  __shared__ U128 red[kPackThreads / 64][3];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) {
#pragma unroll
    for (int ci = 0; ci < 3; ++ci) red[wave][ci] = part[ci];
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    U128 t = {0ull, 0ull};
    for (int wv = 0; wv < kPackThreads / 64; ++wv) add128(t, red[wv][threadIdx.x].lo, red[wv][threadIdx.x].hi);
    uint64_t *dst = reinterpret_cast<uint64_t *>(ws + kWsPartialsOffset) + ((int64_t)blockIdx.x * 3 + threadIdx.x) * 2;
    dst[0] = t.lo;
    dst[1] = t.hi;
  }
}

__global__ void pack_clear_kernel(uint8_t *__restrict__ ws) {
  if (threadIdx.x < kWsPartialsOffset / 4) reinterpret_cast<uint32_t *>(ws)[threadIdx.x] = 0u;
}

// Sum the per-block partials into the three totals (one block).
__global__ __launch_bounds__(kPackThreads) void pack_reduce_kernel(uint8_t *__restrict__ ws, int64_t nblocks) {
  const uint64_t *src = reinterpret_cast<const uint64_t *>(ws + kWsPartialsOffset);
  U128 acc[3] = {{0ull, 0ull}, {0ull, 0ull}, {0ull, 0ull}};
  for (int64_t b = threadIdx.x; b < nblocks; b += kPackThreads) {
#pragma unroll
    for (int ci = 0; ci < 3; ++ci) add128(acc[ci], src[(b * 3 + ci) * 2], src[(b * 3 + ci) * 2 + 1]);
  }
  __shared__ U128 red[kPackThreads / 64][3];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
#pragma unroll
  for (int ci = 0; ci < 3; ++ci) {
    const U128 v = wave_sum128(acc[ci]);
    if (lane == 0) red[wave][ci] = v;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    U128 t = {0ull, 0ull};
    for (int wv = 0; wv < kPackThreads / 64; ++wv) add128(t, red[wv][threadIdx.x].lo, red[wv][threadIdx.x].hi);
    uint64_t *dst = reinterpret_cast<uint64_t *>(ws + kWsTotalsOffset) + threadIdx.x * 2;
    dst[0] = t.lo;
    dst[1] = t.hi;
  }
}

// Nibble slot of element k (0..7) inside a 32-bit vals word: elements
// 0,2,4,6 take slots 0..3 and elements 1,3,5,7 slots 4..7, so that a single
// mask of 0x000F000F (after a shift by 4p) yields elements (2p, 2p+1).
__host__ __device__ constexpr int nibble_slot(int k) { return (k & 1) ? 4 + (k >> 1) : (k >> 1); }

template <int NK, bool HN, bool HG>
__global__ __launch_bounds__(kPackThreads) void pack_emit_kernel(
    const uint16_t *__restrict__ w, ImportanceIn imp, int rows, int cols, int group_size,
    int32_t *__restrict__ row_ptr, uint8_t *__restrict__ vals,
    uint16_t *__restrict__ codes, uint16_t *__restrict__ scales) {
  const int S = cols / kSegCols;
  const int64_t total = (int64_t)rows * S;
  const int64_t f = (int64_t)blockIdx.x * kPackThreads + threadIdx.x;
  const bool valid = f < total;
  const int64_t row = valid ? f / S : 0;
  const int seg = valid ? (int)(f % S) : 0;

  uint32_t kv[16 * NK];
  int kc[16 * NK];
  load_and_select<NK, HN, HG>(w, imp, row, seg, cols, valid, kv, kc);
  // every lane (valid or not) takes part in the shuffles
  const uint32_t s = scale_bits(group_amax(segment_amax<NK>(kv), group_size));
  if (!valid) return;

  const int64_t nnz_row = (int64_t)cols * NK / 4;
  const int64_t e0 = row * nnz_row + (int64_t)seg * 16 * NK;  // first element of the segment

  // vals: 2*NK little-endian 32-bit words
  uint32_t vw[2 * NK];
#pragma unroll
  for (int j = 0; j < 2 * NK; ++j) {
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t u = (uint32_t)(quantize(kv[8 * j + k], s) + 8);
      word |= u << (4 * nibble_slot(k));
    }
    vw[j] = word;
  }
  uint32_t *vdst = reinterpret_cast<uint32_t *>(vals + e0 / 2);
  if constexpr (NK == 1) {
    *reinterpret_cast<uint2 *>(vdst) = make_uint2(vw[0], vw[1]);
  } else if constexpr (NK == 2) {
    *reinterpret_cast<uint4 *>(vdst) = make_uint4(vw[0], vw[1], vw[2], vw[3]);
  } else {
    reinterpret_cast<uint4 *>(vdst)[0] = make_uint4(vw[0], vw[1], vw[2], vw[3]);
    reinterpret_cast<uint4 *>(vdst)[1] = make_uint4(vw[4], vw[5], vw[6], vw[7]);
  }

  // codes: 16*NK two-bit fields, 16 per 32-bit word (two uint16 words)
  if constexpr (NK < 4) {
    uint32_t cw[NK];
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) word |= (uint32_t)kc[16 * j + k] << (2 * k);
      cw[j] = word;
    }
    uint32_t *cdst = reinterpret_cast<uint32_t *>(codes + e0 / 8);
    if constexpr (NK == 1) {
      cdst[0] = cw[0];
    } else {
      *reinterpret_cast<uint2 *>(cdst) = make_uint2(cw[0], cw[1]);
    }
  }

  const int segs_per_group = group_size / kSegCols;
  if (seg % segs_per_group == 0) {
    scales[row * (cols / group_size) + seg / segs_per_group] = (uint16_t)s;
  }
  if (seg == 0) {
    row_ptr[row] = (int32_t)(row * nnz_row);
    if (row == rows - 1) row_ptr[rows] = (int32_t)(rows * nnz_row);
  }
}

template <int NK, bool HN, bool HG>
hipError_t analyze_t(const uint16_t *w, ImportanceIn imp, int32_t rows, int32_t cols, bool adaptive,
                     uint8_t *wsb, hipStream_t stream) {
  hipLaunchKernelGGL((pack_analyze_kernel<NK, HN, HG>), dim3((unsigned)pack_blocks(rows, cols)),
                     dim3(kPackThreads), 0, stream, w, imp, rows, cols, (int)adaptive, wsb);
  return hipGetLastError();
}

template <int NK, bool HN, bool HG>
hipError_t emit_t(const uint16_t *w, ImportanceIn imp, int32_t rows, int32_t cols, int32_t group_size,
                  const i4s_packed &out, hipStream_t stream) {
  hipLaunchKernelGGL((pack_emit_kernel<NK, HN, HG>), dim3((unsigned)pack_blocks(rows, cols)),
                     dim3(kPackThreads), 0, stream, w, imp, rows, cols, group_size, out.row_ptr,
                     out.vals, out.codes, out.scales);
  return hipGetLastError();
}

// Instantiate a launcher for the runtime (n_keep, norms?, gradients?) triple.
template <template <int, bool, bool> class F, typename... A>
hipError_t dispatch_pack(int32_t n_keep, bool hn, bool hg, A... args) {
#define I4S_PACK_NK(NK)                                  \
  if (hn && hg) return F<NK, true, true>::go(args...);   \
  if (hn) return F<NK, true, false>::go(args...);        \
  if (hg) return F<NK, false, true>::go(args...);        \
  return F<NK, false, false>::go(args...);
  switch (n_keep) {
    case 1: { I4S_PACK_NK(1) }
    case 2: { I4S_PACK_NK(2) }
    default: { I4S_PACK_NK(4) }
  }
#undef I4S_PACK_NK
}

template <int NK, bool HN, bool HG>
struct AnalyzeF {
  static hipError_t go(const uint16_t *w, ImportanceIn imp, int32_t rows, int32_t cols, bool adaptive,
                       uint8_t *wsb, hipStream_t stream) {
    return analyze_t<NK, HN, HG>(w, imp, rows, cols, adaptive, wsb, stream);
  }
};

template <int NK, bool HN, bool HG>
struct EmitF {
  static hipError_t go(const uint16_t *w, ImportanceIn imp, int32_t rows, int32_t cols, int32_t group_size,
                       const i4s_packed *out, hipStream_t stream) {
    return emit_t<NK, HN, HG>(w, imp, rows, cols, group_size, *out, stream);
  }
};

}  // namespace

hipError_t launch_pack_analyze(const uint16_t *w, const float *col_norm, const uint16_t *grad,
                               int32_t rows, int32_t cols, int32_t n_keep, bool adaptive, void *ws,
                               hipStream_t stream) {
  uint8_t *wsb = static_cast<uint8_t *>(ws);
  // the flag and the totals start at zero (a fill kernel, not a memset node)
  hipLaunchKernelGGL(pack_clear_kernel, dim3(1), dim3(64), 0, stream, wsb);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const ImportanceIn imp = {col_norm, grad};
  err = dispatch_pack<AnalyzeF>(n_keep, col_norm != nullptr, grad != nullptr, w, imp, rows, cols,
                                adaptive, wsb, stream);
  if (err != hipSuccess || !adaptive) return err;
  hipLaunchKernelGGL(pack_reduce_kernel, dim3(1), dim3(kPackThreads), 0, stream, wsb,
                     pack_blocks(rows, cols));
  return hipGetLastError();
}

hipError_t launch_pack_emit(const uint16_t *w, const float *col_norm, const uint16_t *grad,
                            int32_t rows, int32_t cols, int32_t n_keep, int32_t group_size,
                            const i4s_packed &out, hipStream_t stream) {
  const ImportanceIn imp = {col_norm, grad};
  return dispatch_pack<EmitF>(n_keep, col_norm != nullptr, grad != nullptr, w, imp, rows, cols,
                              group_size, &out, stream);
}

}  // namespace i4s
