// Floor measurements for the SparseGEMV benchmark (libi4s_floor.so).
//
// Not part of the libi4s ABI: two reference kernels that the benchmark times
// the same way as the GEMV, so that its bandwidth figure can be read against
// what one launch of this size can reach on the part at all.
//
//   i4sf_stream_read: one launch that reads `bytes` (a multiple of 16) once,
//     every lane one 16-byte load, 256 lanes per block; optionally with
//     nontemporal loads.  Nothing is written unless the data hash to a value
//     the caller's fill cannot produce.
//   i4sf_chase: one lane follows `steps` dependent loads through `next`
//     (idx = next[idx], starting at 0) and stores the last index; elapsed
//     time / steps is the latency of one load that misses every cache when
//     the chain is spread over more memory than the caches hold.
//
// Both return 0 on success, 1 on a bad argument (checked before launching),
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

__global__ void chase_kernel(const uint32_t *__restrict__ next, uint64_t n, int32_t steps,
                             uint32_t *__restrict__ out) {
  uint32_t j = 0;
  for (int32_t s = 0; s < steps; ++s) {
    j = __builtin_nontemporal_load(next + j);
    if (j >= n) break;  // a chain that leaves the buffer stops here
  }
  out[0] = j;
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

int i4sf_chase(const uint32_t *next, uint64_t n, int32_t steps, uint32_t *out, void *stream) {
  if (!next || !out || n == 0 || n > 0xFFFFFFFFull || steps < 1) return 1;
  hipLaunchKernelGGL(chase_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream), next, n, steps, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
