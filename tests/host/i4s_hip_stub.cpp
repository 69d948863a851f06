// Stand-ins for the HIP runtime calls and the kernel launchers that the host
// layer of libi4s (i4s_api.cpp) makes, so that the host layer can be built
// for the CPU alone -- with AddressSanitizer and UndefinedBehaviorSanitizer --
// and its argument checks, error paths and decisions exercised without a GPU.
//
// Here "device" memory is host memory.  No kernel runs: a launch is counted
// and its arguments are kept for the driver to inspect.  The device reports
// the architecture the driver sets (gfx950 unless told otherwise), which is
// how a test forces I4S_ERR_UNSUPPORTED.  The pack analysis writes the flag
// word and the three SSE totals the driver chose into the workspace, where
// the host layer reads them back.  Test infrastructure only.

#include <hip/hip_runtime.h>

#include <cstring>

#include "i4s_internal.h"
#include "i4s_hip_stub.h"

namespace {

char g_arch[64] = "gfx950";
int g_launches = 0;
uint32_t g_pack_flag = 0;
uint64_t g_totals[6] = {};
i4s_stub_launch g_last = {};
alignas(256) unsigned char g_scratch[1024];

}  // namespace

extern "C" {

void i4s_stub_set_arch(const char *arch) {
  std::strncpy(g_arch, arch, sizeof(g_arch) - 1);
  g_arch[sizeof(g_arch) - 1] = '\0';
}

void i4s_stub_set_pack_result(uint32_t flag, const uint64_t totals_lo_hi[6]) {
  g_pack_flag = flag;
  std::memcpy(g_totals, totals_lo_hi, sizeof(g_totals));
}

int i4s_stub_launches(void) { return g_launches; }

i4s_stub_launch i4s_stub_last_launch(void) { return g_last; }

const void *i4s_stub_scratch(void) { return g_scratch; }

hipError_t hipGetDevice(int *device) {
  *device = 0;
  return hipSuccess;
}

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *prop, int device) {
  (void)device;
  std::memset(prop, 0, sizeof(*prop));
  std::strncpy(prop->gcnArchName, g_arch, sizeof(prop->gcnArchName) - 1);
  return hipSuccess;
}

const char *hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }

hipError_t hipMemcpyAsync(void *dst, const void *src, size_t bytes, hipMemcpyKind kind, hipStream_t stream) {
  (void)kind;
  (void)stream;
  std::memcpy(dst, src, bytes);
  return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t stream) {
  (void)stream;
  return hipSuccess;
}

}  // extern "C"

namespace i4s {

hipError_t launch_pack_analyze(const uint16_t *w, const float *col_norm, const uint16_t *grad, int32_t rows,
                               int32_t cols, int32_t n_keep, bool adaptive, void *ws, hipStream_t stream) {
  (void)w, (void)col_norm, (void)grad, (void)stream;
  ++g_launches;
  g_last = {};
  g_last.kind = 1;
  g_last.rows = rows;
  g_last.cols = cols;
  g_last.n_keep = n_keep;
  g_last.adaptive = adaptive;
  unsigned char *p = static_cast<unsigned char *>(ws);
  std::memcpy(p + kWsFlagOffset, &g_pack_flag, 4);
  std::memcpy(p + kWsTotalsOffset, g_totals, sizeof(g_totals));
  return hipSuccess;
}

hipError_t launch_pack_emit(const uint16_t *w, const float *col_norm, const uint16_t *grad, int32_t rows,
                            int32_t cols, int32_t n_keep, int32_t group_size, const i4s_packed &out,
                            hipStream_t stream) {
  (void)w, (void)col_norm, (void)grad, (void)out, (void)stream;
  ++g_launches;
  g_last = {};
  g_last.kind = 2;
  g_last.rows = rows;
  g_last.cols = cols;
  g_last.n_keep = n_keep;
  g_last.group_size = group_size;
  return hipSuccess;
}

static hipError_t record_gemv(int kind, const i4s_packed &w, int32_t batch, const void *workspace) {
  ++g_launches;
  g_last = {};
  g_last.kind = kind;
  g_last.rows = w.rows;
  g_last.cols = w.cols;
  g_last.n_keep = w.n_keep;
  g_last.group_size = w.group_size;
  g_last.batch = batch;
  g_last.workspace = workspace;
  return hipSuccess;
}

hipError_t launch_gemv(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y, hipStream_t stream) {
  (void)x, (void)y, (void)stream;
  return record_gemv(3, w, batch, nullptr);
}

hipError_t launch_gemv_ws(const i4s_packed &w, const uint16_t *x, int32_t batch, uint16_t *y,
                          const SplitPlan &plan, void *workspace, hipStream_t stream) {
  (void)x, (void)y, (void)plan, (void)stream;
  return record_gemv(4, w, batch, workspace);
}

hipError_t launch_gemv_multi(const i4s_packed *w, int32_t n, const uint16_t *x, int32_t batch, uint16_t *const *y,
                             hipStream_t stream) {
  (void)x, (void)y, (void)stream;
  const hipError_t e = record_gemv(5, w[0], batch, nullptr);
  g_last.layers = n;
  return e;
}

hipError_t noalloc_scratch(void **ptr) {
  *ptr = g_scratch;
  return hipSuccess;
}

}  // namespace i4s
