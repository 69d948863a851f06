// Floor measurements for the SparseGEMV benchmark (libi4s_floor.so).
//
// Not part of the libi4s ABI: reference kernels that the benchmark times the
// same way as the GEMV, so that its bandwidth figure can be read against what
// one launch of this size can reach on the part at all, plus a bounded delay
// kernel that lets the benchmark queue a whole timed sequence before the GPU
// starts on it.
//
//   i4sf_stream_read: one launch that reads `bytes` (a multiple of 16) once,
//     every lane one 16-byte load, 256 lanes per block; optionally with
//     nontemporal loads.  Nothing is written unless the data hash to a value
//     the caller's fill cannot produce.
//   i4sf_stream_read_shape: the same read with a chosen shape: `vpl`
//     16-byte loads per lane (1, 2, 4 or 8; all issued before the first
//     use, lane-contiguous within each block-wide slab so every load
//     instruction is coalesced), `threads` per block (64..1024, a multiple
//     of 64), and either one block per slab (`blocks` = 0) or a fixed grid
//     of `blocks` blocks that stride over the slabs (a persistent grid).
//   i4sf_chase: one lane follows `steps` dependent loads through `next`
//     (idx = next[idx], starting at 0) and stores the last index; elapsed
//     time / steps is the latency of one load that misses every cache when
//     the chain is spread over more memory than the caches hold.
//   i4sf_delay: one wave that sleeps until `microseconds` of the GPU's
//     constant real-time clock have passed (bounded by an iteration cap as
//     well, so it always ends), then exits.  Enqueued ahead of a timed
//     sequence it keeps the queue busy while the host submits that sequence.
//
// All return 0 on success, 1 on a bad argument (checked before launching),
// 2 when the launch fails.  Pointers are device pointers; `stream` is a
// hipStream_t.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t *__restrict__ p, uint64_t n,
                                                          uint32_t *__restrict__ sink) {
  const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const u32x4_t v = NT ? __builtin_nontemporal_load(p + i) : p[i];
  const uint32_t h = v.x ^ v.y ^ v.z ^ v.w;
  if (h == 0x9E3779B9u) sink[0] = h;
}

// Slab s covers vectors [s * blockDim * VPL, (s + 1) * blockDim * VPL); load
// j of thread t reads vector s * blockDim * VPL + j * blockDim + t, clamped to
// the last vector (re-reading it is harmless).  A block handles slabs
// blockIdx.x, blockIdx.x + gridDim.x, ... (one slab when the grid covers all).
template <int VPL>
__global__ __launch_bounds__(1024) void stream_read_shape_kernel(const u32x4_t *__restrict__ p, uint64_t n,
                                                                 uint64_t slabs, uint32_t *__restrict__ sink) {
  const uint64_t per = (uint64_t)blockDim.x * VPL;
  uint32_t h = 0;
  for (uint64_t s = blockIdx.x; s < slabs; s += gridDim.x) {
    u32x4_t v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      uint64_t i = s * per + (uint64_t)j * blockDim.x + threadIdx.x;
      i = i < n ? i : n - 1;
      v[j] = __builtin_nontemporal_load(p + i);
    }
#pragma unroll
    for (int j = 0; j < VPL; ++j) h ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (h == 0x9E3779B9u) sink[0] = h;
}

__global__ void chase_kernel(const uint32_t *__restrict__ next, uint64_t n, int32_t steps,
                             uint32_t *__restrict__ out) {
  uint32_t j = 0;
  for (int32_t s = 0; s < steps; ++s) {
    j = __builtin_nontemporal_load(next + j);
    if (j >= n) break;  // a chain that leaves the buffer stops here
  }
  out[0] = j;
}

// s_memrealtime counts at a constant 100 MHz on this GPU family.  The loop
// also stops after max_iter sleeps, whatever the clock reads.
__global__ void delay_kernel(uint64_t ticks, uint32_t max_iter) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t it = 0; it < max_iter; ++it) {
    if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(16);
  }
}

}  // namespace

extern "C" {

int i4sf_stream_read(const void *p, uint64_t bytes, int nontemporal, uint32_t *sink, void *stream) {
  if (!p || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)p & 15) != 0) return 1;
  const uint64_t n = bytes / 16;
  const uint64_t blocks = (n + 255) / 256;
  if (blocks > 0x7FFFFFFFull) return 1;
  const u32x4_t *q = static_cast<const u32x4_t *>(p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, q, n, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, q, n, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int i4sf_stream_read_shape(const void *p, uint64_t bytes, int vpl, int threads, int blocks, uint32_t *sink,
                           void *stream) {
  if (!p || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)p & 15) != 0) return 1;
  if (vpl != 1 && vpl != 2 && vpl != 4 && vpl != 8) return 1;
  if (threads < 64 || threads > 1024 || threads % 64 != 0 || blocks < 0) return 1;
  const uint64_t n = bytes / 16;
  const uint64_t per = (uint64_t)threads * vpl;
  const uint64_t slabs = (n + per - 1) / per;
  const uint64_t grid = blocks > 0 ? (uint64_t)blocks : slabs;
  if (grid == 0 || grid > 0x7FFFFFFFull) return 1;
  const u32x4_t *q = static_cast<const u32x4_t *>(p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g((unsigned)grid), b((unsigned)threads);
  switch (vpl) {
    case 1: hipLaunchKernelGGL(stream_read_shape_kernel<1>, g, b, 0, st, q, n, slabs, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_shape_kernel<2>, g, b, 0, st, q, n, slabs, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_shape_kernel<4>, g, b, 0, st, q, n, slabs, sink); break;
    default: hipLaunchKernelGGL(stream_read_shape_kernel<8>, g, b, 0, st, q, n, slabs, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int i4sf_chase(const uint32_t *next, uint64_t n, int32_t steps, uint32_t *out, void *stream) {
  if (!next || !out || n == 0 || n > 0xFFFFFFFFull || steps < 1) return 1;
  hipLaunchKernelGGL(chase_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream), next, n, steps, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int i4sf_delay(uint32_t microseconds, void *stream) {
  if (microseconds == 0 || microseconds > 100000) return 1;  // at most 0.1 s
  const uint64_t ticks = (uint64_t)microseconds * 100;      // 100 MHz real-time clock
  // s_sleep 16 is about 1024 clocks (~0.4 us at 2.4 GHz): the cap allows
  // several times the requested span before the loop gives up
  const uint32_t max_iter = microseconds * 20 + 1000;
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ticks, max_iter);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
