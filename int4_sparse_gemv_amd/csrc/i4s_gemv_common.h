// Device helpers shared by the GEMV kernels of libi4s (gfx950).  Internal.
//
// Method: "Efficient LLM-based Advertising via Model Compression and Parallel
// Verification", section 3.3, "Computational Acceleration": INT4 weights are
// widened to fp16 with a few bit operations and the 2-bit indices packed in
// uint16 words are decoded with shifts and masks.  The helpers below are
// written for CDNA4 (wave64, v_and_or_b32, v_perm_b32, DPP), not taken from
// the page's NVIDIA kernel.
//
// Per 8 stored elements (one 32-bit vals word) the decode is one shift, four
// v_and_or_b32 that drop nibble pairs into the mantissa of 1024.0 (fp16
// 0x6400) and four packed fp16 adds/fmas that remove the bias exactly; the
// nibble interleave of the format puts elements (2p, 2p+1) in bits 4p and
// 16+4p so one mask yields one pair.  For 2:4, a group's 4-bit code picks a
// v_perm_b32 selector that moves the two kept activations out of the group's
// four into one fp16 pair.  Row sums across lanes use DPP row rotations and
// four lane reads (no LDS traffic).
#pragma once

#include "i4s_internal.h"

namespace i4s {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLdsBudget = 64 * 1024;  // bytes of LDS for staged activations
constexpr int kStrideB1 = 72;          // halfs per unit, batch-1 kernel (16-byte reads)
constexpr int kStrideBT = 68;          // halfs per unit, batch kernel (8-byte reads)

__device__ inline h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }

// (a & m) | c in one VALU op; GFX9 VOP3 takes no literal, so m comes in an SGPR.
__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(m), "v"(c));
  return d;
}

// Four exact fp16 pairs (q_{2p}, q_{2p+1}), p = 0..3, of one vals word.
__device__ inline void dequant_word(uint32_t w, h2_t q[4]) {
  const uint32_t magic = 0x64006400u;  // 1024.0 in both halves
  const uint32_t t = w >> 8;
  const h2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2_t bias16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  // slots 0/4 and 2/6: nibble in mantissa bits 0..3 -> 1024 + u
  q[0] = as_h2(and_or(w, 0x000F000Fu, magic)) + bias;
  q[2] = as_h2(and_or(t, 0x000F000Fu, magic)) + bias;
  // slots 1/5 and 3/7: nibble in mantissa bits 4..7 -> 1024 + 16u
  q[1] = __builtin_elementwise_fma(as_h2(and_or(w, 0x00F000F0u, magic)), sixteenth, bias16);
  q[3] = __builtin_elementwise_fma(as_h2(and_or(t, 0x00F000F0u, magic)), sixteenth, bias16);
}

// v_perm_b32 selector taking fp16 lanes cf and cs of a group's four
// activations (held as two dwords {x0|x1<<16, x2|x3<<16}) into (lo, hi):
// bytes [2cf, 2cf+1, 2cs, 2cs+1], for the code nibble h = cf | cs << 2.
// The multiply spreads the two 2-bit fields into four byte lanes without
// carries between them.
__host__ __device__ constexpr uint32_t pair_selector(uint32_t h) {
  return ((h * 0x808202u) & 0x06060606u) | 0x01000100u;
}

// 1:4: a pair of stored elements (2k, 2k+1) belongs to groups 2k and 2k+1,
// each keeping one column; their codes form nibble h = cA | cB << 2.  Two
// v_perm_b32 selectors move activation cA of group 2k into the low half and
// activation cB of group 2k+1 into the high half (selector byte 0x0C gives
// a zero byte), so an OR of the two results is the activation pair.
__host__ __device__ constexpr uint32_t single_selector_lo(uint32_t c) {
  return (2 * c) | ((2 * c + 1) << 8) | 0x0C0C0000u;
}
__host__ __device__ constexpr uint32_t single_selector_hi(uint32_t c) {
  return 0x00000C0Cu | ((2 * c) << 16) | ((2 * c + 1) << 24);
}

// Hides a value's origin from the optimizer.  Selector-table offsets are
// built once per code dword as four byte lanes and then taken out one byte at
// a time (one v_bfe_u32 each); without this the compiler folds the masks back
// into every extraction and spends a shift and an AND per group.
__device__ inline void opaque(uint32_t &v) { asm("" : "+v"(v)); }

// Keeps the loads issued before it ahead of those issued after it: the empty
// asm with a memory clobber stops the IR passes from sinking loads towards
// their first use, and the scheduling barrier does the same for the machine
// scheduler.  (No wait is implied: nothing reads the loaded registers.)
__device__ inline void issue_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ inline float fp16_bits_to_float(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// float -> fp16 bits, round to nearest even
__device__ inline uint32_t float_to_fp16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int CTRL>
__device__ inline float dpp_rot_add(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
  return v + __builtin_bit_cast(float, s);
}

// Sum over the 64 lanes; every lane gets the result.  Rotations by 8, 4, 2,
// 1 inside each 16-lane row (DPP row_ror), then the four row sums.
__device__ inline float wave_sum(float v) {
  v = dpp_rot_add<0x128>(v);
  v = dpp_rot_add<0x124>(v);
  v = dpp_rot_add<0x122>(v);
  v = dpp_rot_add<0x121>(v);
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

template <int NK>
struct UnitRegs {
  uint32_t v[2 * NK];                 // vals words of the unit
  uint32_t c[NK < 4 ? NK : 1];        // code dwords (16 codes each)
  uint32_t s;                         // scale bits
};

// Loads one unit: elem0 is the unit's first element (row start + 16*NK*u).
template <int NK>
__device__ inline void load_unit(UnitRegs<NK> &r, const uint8_t *__restrict__ vals,
                                 const uint16_t *__restrict__ codes,
                                 const uint16_t *__restrict__ scales, uint32_t elem0,
                                 uint32_t scale_idx) {
  const uint32_t *vp = reinterpret_cast<const uint32_t *>(vals + (elem0 >> 1));
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
    r.c[0] = *reinterpret_cast<const uint32_t *>(codes + (elem0 >> 3));
  } else if constexpr (NK == 2) {
    const uint2 c = *reinterpret_cast<const uint2 *>(codes + (elem0 >> 3));
    r.c[0] = c.x; r.c[1] = c.y;
  }
  r.s = *reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(scales) + 2u * scale_idx);
}

// Fill the 16-entry selector table (2:4 only); call with threadIdx.x < 16.
__device__ inline void init_selector_table(uint32_t *lut) {
  lut[threadIdx.x] = pair_selector(threadIdx.x);
}

__device__ inline uint32_t lut_read(const uint32_t *lut, uint32_t byte_off) {
  return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lut) + byte_off);
}

// Fill the 16-entry table of 1:4 selector pairs (32 words, 8-byte aligned);
// call with threadIdx.x < 16.
__device__ inline void init_single_table(uint32_t *lut) {
  lut[2 * threadIdx.x] = single_selector_lo(threadIdx.x & 3u);
  lut[2 * threadIdx.x + 1] = single_selector_hi(threadIdx.x >> 2);
}

typedef uint32_t u32x2_lut_t __attribute__((ext_vector_type(2)));

// The selector pair at byte offset 8 * h.
__device__ inline u32x2_lut_t lut_read2(const uint32_t *lut, uint32_t byte_off) {
  return *reinterpret_cast<const u32x2_lut_t *>(reinterpret_cast<const char *>(lut) + byte_off);
}

// Fill whichever selector table pattern NK uses (none for dense).
template <int NK>
__device__ inline void init_tables(uint32_t *lut) {
  if constexpr (NK == 2) {
    if (threadIdx.x < 16) init_selector_table(lut);
  } else if constexpr (NK == 1) {
    if (threadIdx.x < 16) init_single_table(lut);
  }
}

// A row start read from row_ptr, made safe to use as an offset: clamped to
// [0, last_start] (last_start = (rows - 1) * nnz_row, the start of the last
// row) and aligned down to a whole 64-column unit (16 * NK elements).  A
// descriptor that meets the documented precondition passes unchanged; one
// that does not reads inside the buffers (and gives unspecified values)
// instead of reading out of bounds.  Used only on the rare path of a row
// stored away from the format's offset.
template <int NK>
__device__ inline uint32_t safe_row_start(int32_t rp, uint32_t last_start) {
  const uint32_t v = rp < 0 ? 0u : (uint32_t)rp;
  return (v < last_start ? v : last_start) & ~(16u * NK - 1u);
}

// Orders the LDS accesses of one wave around an exchange between its own
// lanes (a lane writes, other lanes of the same wave read, or the area is
// rewritten after such reads): everything a lane wrote before it is seen by
// every lane of the wave after it, and no LDS access of the wave moves
// across it.  Wavefront-scope fences restricted to LDS around a wave
// barrier.  A wave's LDS operations complete in program order, so on this
// ISA it emits no instruction; what it adds is that the compiler may no
// longer move the accesses of different lanes past one another, which the
// language otherwise allows for accesses that race between lanes.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Block barrier that orders LDS only: the fences are restricted to the local
// address space, so no wave waits here for its outstanding global loads.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// The two halves of load_unit_nt, for kernels that issue every unit's codes
// before any unit's vals (the codes of 2:4 and 1:4 only).
template <int NK>
__device__ inline void load_codes_nt(UnitRegs<NK> &r, const uint16_t *__restrict__ codes, uint32_t elem0) {
  if constexpr (NK == 1) {
    r.c[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(codes + (elem0 >> 3)));
  } else if constexpr (NK == 2) {
    const u32x2_t c = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(codes + (elem0 >> 3)));
    r.c[0] = c.x; r.c[1] = c.y;
  }
}
template <int NK>
__device__ inline void load_vals_scale_nt(UnitRegs<NK> &r, const uint8_t *__restrict__ vals,
                                          const uint16_t *__restrict__ scales, uint32_t elem0, uint32_t scale_idx) {
  const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(vals + (elem0 >> 1));
  if constexpr (NK == 1) {
    const u32x2_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(vp));
    r.v[0] = a.x; r.v[1] = a.y;
  } else {
    const u32x4_t a = __builtin_nontemporal_load(vp);
    r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
  }
  r.s = __builtin_nontemporal_load(
      reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(scales) + 2u * scale_idx));
}

template <int NK>
__device__ inline void load_unit_nt(UnitRegs<NK> &r, const uint8_t *__restrict__ vals,
                                    const uint16_t *__restrict__ codes,
                                    const uint16_t *__restrict__ scales, uint32_t elem0,
                                    uint32_t scale_idx) {
  const u32x4_t *vp = reinterpret_cast<const u32x4_t *>(vals + (elem0 >> 1));
  if constexpr (NK == 1) {
    const u32x2_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(vp));
    r.v[0] = a.x; r.v[1] = a.y;
  } else if constexpr (NK == 2) {
    const u32x4_t a = __builtin_nontemporal_load(vp);
    r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
  } else {
    const u32x4_t a = __builtin_nontemporal_load(vp);
    const u32x4_t b = __builtin_nontemporal_load(vp + 1);
    r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
    r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
  }
  if constexpr (NK == 1) {
    r.c[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(codes + (elem0 >> 3)));
  } else if constexpr (NK == 2) {
    const u32x2_t c = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(codes + (elem0 >> 3)));
    r.c[0] = c.x; r.c[1] = c.y;
  }
  r.s = __builtin_nontemporal_load(
      reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(scales) + 2u * scale_idx));
}

}  // namespace
}  // namespace i4s
