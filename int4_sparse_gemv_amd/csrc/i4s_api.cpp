// Host layer of libi4s: argument validation, device check, kernel dispatch
// and status reporting for the C ABI declared in include/i4s.h.
//
// Every check runs before anything is enqueued.  Nothing here allocates
// device memory: buffers and the pack workspace belong to the caller.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "i4s.h"
#include "i4s_internal.h"

namespace {

thread_local std::string g_last_error;

i4s_status fail(i4s_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

i4s_status device_error(hipError_t e, const char *what) {
  return fail(I4S_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// Shape/pattern checks shared by pack_sizes, pack and run.  `allow_adaptive`
// admits group_size 0 (pack only).
i4s_status check_shape(int32_t rows, int32_t cols, int32_t n_keep, int32_t group_size,
                       bool allow_adaptive) {
  if (rows < 1) return fail(I4S_ERR_INVALID_ARGUMENT, "rows=%d must be >= 1", rows);
  if (cols < i4s::kSegCols || cols % i4s::kSegCols)
    return fail(I4S_ERR_INVALID_ARGUMENT, "cols=%d must be a positive multiple of 64", cols);
  if (n_keep != 1 && n_keep != 2 && n_keep != 4)
    return fail(I4S_ERR_INVALID_ARGUMENT, "n_keep=%d must be 1, 2 or 4", n_keep);
  if (group_size == 0) {
    if (!allow_adaptive) return fail(I4S_ERR_INVALID_ARGUMENT, "group_size 0 (adaptive) is only valid for packing");
    if (cols % 256)
      return fail(I4S_ERR_INVALID_ARGUMENT, "adaptive group size needs cols=%d to be a multiple of 256", cols);
  } else if (group_size != 64 && group_size != 128 && group_size != 256) {
    return fail(I4S_ERR_INVALID_ARGUMENT, "group_size=%d must be 64, 128, 256 or 0", group_size);
  } else if (cols % group_size) {
    return fail(I4S_ERR_INVALID_ARGUMENT, "cols=%d is not a multiple of group_size=%d", cols, group_size);
  }
  const int64_t nnz = (int64_t)rows * cols / 4 * n_keep;
  if (nnz >= (int64_t(1) << 31))
    return fail(I4S_ERR_INVALID_ARGUMENT, "rows*cols*n_keep/4 = %lld does not fit int32 row pointers",
                (long long)nnz);
  return I4S_OK;
}

// gfx950 only.  The answer per device is cached (a benign, monotonic cache).
std::atomic<int> g_arch_ok[64];

i4s_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error(e, "hipGetDevice");
  if (dev >= 0 && dev < 64) {
    const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return I4S_OK;
    if (c == 2) return fail(I4S_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return device_error(e, "hipGetDeviceProperties");
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  if (!ok) return fail(I4S_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return I4S_OK;
}

struct U128 {
  uint64_t lo, hi;
};
bool less128(const U128 &a, const U128 &b) { return a.hi < b.hi || (a.hi == b.hi && a.lo < b.lo); }

}  // namespace

extern "C" {

i4s_status i4s_pack_sizes(int32_t rows, int32_t cols, int32_t n_keep, int32_t group_size,
                          i4s_sizes *out) {
  if (!out) return fail(I4S_ERR_INVALID_ARGUMENT, "out is NULL");
  const i4s_status st = check_shape(rows, cols, n_keep, group_size, true);
  if (st != I4S_OK) return st;
  const uint64_t nnz = (uint64_t)rows * cols / 4 * n_keep;
  const int32_t g_min = group_size == 0 ? 64 : group_size;
  out->row_ptr = 4ull * ((uint64_t)rows + 1);
  out->vals = nnz / 2;
  out->codes = n_keep < 4 ? nnz / 4 : 0;
  out->scales = 2ull * rows * (uint64_t)(cols / g_min);
  out->workspace = i4s::pack_workspace_bytes(rows, cols);
  return I4S_OK;
}

i4s_status i4s_pack(const uint16_t *w_fp16, int32_t rows, int32_t cols, int32_t n_keep,
                    int32_t group_size, void *workspace, uint64_t workspace_bytes,
                    i4s_packed *inout, i4s_pack_report *report, void *stream) {
  return i4s_pack_ex(w_fp16, rows, cols, n_keep, group_size, nullptr, nullptr, workspace,
                     workspace_bytes, inout, report, stream);
}

i4s_status i4s_pack_ex(const uint16_t *w_fp16, int32_t rows, int32_t cols, int32_t n_keep,
                       int32_t group_size, const float *col_norm, const uint16_t *grad_fp16,
                       void *workspace, uint64_t workspace_bytes, i4s_packed *inout,
                       i4s_pack_report *report, void *stream) {
  i4s_sizes sz;
  i4s_status st = i4s_pack_sizes(rows, cols, n_keep, group_size, &sz);
  if (st != I4S_OK) return st;
  if (!w_fp16 || !aligned(w_fp16, 16)) return fail(I4S_ERR_INVALID_ARGUMENT, "w_fp16 is NULL or not 16-byte aligned");
  if (col_norm && !aligned(col_norm, 16)) return fail(I4S_ERR_INVALID_ARGUMENT, "col_norm is not 16-byte aligned");
  if (grad_fp16 && !aligned(grad_fp16, 16)) return fail(I4S_ERR_INVALID_ARGUMENT, "grad_fp16 is not 16-byte aligned");
  if (!inout) return fail(I4S_ERR_INVALID_ARGUMENT, "inout is NULL");
  if (!inout->row_ptr || !aligned(inout->row_ptr, 16) || !inout->vals || !aligned(inout->vals, 16) ||
      !inout->scales || !aligned(inout->scales, 16))
    return fail(I4S_ERR_INVALID_ARGUMENT, "row_ptr, vals and scales must be non-NULL and 16-byte aligned");
  if (n_keep < 4 && (!inout->codes || !aligned(inout->codes, 16)))
    return fail(I4S_ERR_INVALID_ARGUMENT, "codes must be non-NULL and 16-byte aligned when n_keep < 4");
  if (!workspace || !aligned(workspace, 16)) return fail(I4S_ERR_INVALID_ARGUMENT, "workspace is NULL or not 16-byte aligned");
  if (workspace_bytes < sz.workspace)
    return fail(I4S_ERR_WORKSPACE_TOO_SMALL, "workspace has %llu bytes, %llu needed",
                (unsigned long long)workspace_bytes, (unsigned long long)sz.workspace);
  {
    // the four outputs and the workspace are written while W and the
    // importance inputs are read: no two of them may share a byte
    const uint64_t wb = 2ull * rows * (uint64_t)cols;
    struct Span {
      const void *p;
      uint64_t n;
      const char *name;
    } span[] = {
        {inout->row_ptr, sz.row_ptr, "row_ptr"}, {inout->vals, sz.vals, "vals"},
        {n_keep < 4 ? inout->codes : nullptr, sz.codes, "codes"}, {inout->scales, sz.scales, "scales"},
        {workspace, sz.workspace, "workspace"},
    };
    const Span in[] = {{w_fp16, wb, "w_fp16"}, {col_norm, 4ull * cols, "col_norm"}, {grad_fp16, wb, "grad_fp16"}};
    const int nspan = (int)(sizeof(span) / sizeof(span[0]));
    for (int i = 0; i < nspan; ++i) {
      if (!span[i].p) continue;
      for (int j = i + 1; j < nspan; ++j)
        if (span[j].p && overlap(span[i].p, span[i].n, span[j].p, span[j].n))
          return fail(I4S_ERR_INVALID_ARGUMENT, "%s and %s overlap", span[i].name, span[j].name);
      for (const Span &r : in)
        if (r.p && overlap(span[i].p, span[i].n, r.p, r.n))
          return fail(I4S_ERR_INVALID_ARGUMENT, "%s overlaps %s", span[i].name, r.name);
    }
  }
  st = check_device();
  if (st != I4S_OK) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool adaptive = group_size == 0;
  hipError_t e = i4s::launch_pack_analyze(w_fp16, col_norm, grad_fp16, rows, cols, n_keep, adaptive, workspace, s);
  if (e != hipSuccess) return device_error(e, "pack analyze launch");
  uint64_t head[i4s::kWsPartialsOffset / 8];
  e = hipMemcpyAsync(head, workspace, sizeof(head), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return device_error(e, "pack read-back");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return device_error(e, "pack synchronize");
  uint32_t flag;
  std::memcpy(&flag, reinterpret_cast<const uint8_t *>(head) + i4s::kWsFlagOffset, 4);
  if (flag & i4s::kPackFlagNonfiniteWeight) return fail(I4S_ERR_NONFINITE_WEIGHT, "W holds an Inf or NaN");
  if (flag & i4s::kPackFlagBadNorm)
    return fail(I4S_ERR_INVALID_ARGUMENT, "col_norm holds a negative, infinite or NaN value");
  if (flag & i4s::kPackFlagBadGrad) return fail(I4S_ERR_INVALID_ARGUMENT, "grad_fp16 holds an Inf or NaN");

  U128 sse[3] = {};
  int32_t g = group_size;
  if (adaptive) {
    const uint64_t *tot = head + i4s::kWsTotalsOffset / 8;
    for (int ci = 0; ci < 3; ++ci) sse[ci] = {tot[2 * ci], tot[2 * ci + 1]};
    int best = 2;  // ties go to the larger group
    for (int ci = 1; ci >= 0; --ci)
      if (less128(sse[ci], sse[best])) best = ci;
    g = 64 << best;
  }
  i4s_packed out = *inout;
  out.rows = rows;
  out.cols = cols;
  out.n_keep = n_keep;
  out.group_size = g;
  out.nnz = (int64_t)rows * cols / 4 * n_keep;
  if (n_keep == 4) out.codes = nullptr;
  e = i4s::launch_pack_emit(w_fp16, col_norm, grad_fp16, rows, cols, n_keep, g, out, s);
  if (e != hipSuccess) return device_error(e, "pack emit launch");
  *inout = out;
  if (report) {
    std::memset(report, 0, sizeof(*report));
    report->group_size = g;
    report->n_candidates = adaptive ? 3 : 0;
    for (int ci = 0; ci < 3; ++ci) {
      report->candidates[ci] = 64 << ci;
      report->sse_lo[ci] = sse[ci].lo;
      report->sse_hi[ci] = sse[ci].hi;
    }
  }
  return I4S_OK;
}

}  // extern "C"

namespace {

// Checks shared by i4s_run, i4s_run_ws and i4s_run_workspace_size.
i4s_status validate_layer(const i4s_packed *w, int32_t batch) {
  if (!w) return fail(I4S_ERR_INVALID_ARGUMENT, "w is NULL");
  i4s_status st = check_shape(w->rows, w->cols, w->n_keep, w->group_size, false);
  if (st != I4S_OK) return st;
  const int64_t nnz = (int64_t)w->rows * w->cols / 4 * w->n_keep;
  if (w->nnz != nnz)
    return fail(I4S_ERR_INVALID_ARGUMENT, "nnz=%lld does not match rows*cols*n_keep/4=%lld",
                (long long)w->nnz, (long long)nnz);
  if (batch < 1 || batch > I4S_MAX_BATCH)
    return fail(I4S_ERR_INVALID_ARGUMENT, "batch=%d must be in [1, %d]", batch, I4S_MAX_BATCH);
  return I4S_OK;
}

i4s_status validate_run(const i4s_packed *w, const uint16_t *x_fp16, int32_t batch, const uint16_t *y_fp16) {
  i4s_status st = validate_layer(w, batch);
  if (st != I4S_OK) return st;
  const int64_t nnz = w->nnz;
  if (!w->row_ptr || !aligned(w->row_ptr, 4) || !w->vals || !aligned(w->vals, 16) || !w->scales ||
      !aligned(w->scales, 2))
    return fail(I4S_ERR_INVALID_ARGUMENT, "row_ptr/vals/scales NULL or misaligned (need 4/16/2 bytes)");
  if (w->n_keep < 4 && (!w->codes || !aligned(w->codes, 8)))
    return fail(I4S_ERR_INVALID_ARGUMENT, "codes NULL or not 8-byte aligned");
  if (!x_fp16 || !aligned(x_fp16, 16)) return fail(I4S_ERR_INVALID_ARGUMENT, "x is NULL or not 16-byte aligned");
  if (!y_fp16 || !aligned(y_fp16, 2)) return fail(I4S_ERR_INVALID_ARGUMENT, "y is NULL or not 2-byte aligned");
  const uint64_t xb = 2ull * batch * w->cols, yb = 2ull * batch * w->rows;
  if (overlap(x_fp16, xb, y_fp16, yb)) return fail(I4S_ERR_INVALID_ARGUMENT, "x and y overlap");
  if (overlap(y_fp16, yb, w->vals, (uint64_t)nnz / 2) ||
      overlap(y_fp16, yb, w->scales, 2ull * w->rows * (w->cols / w->group_size)) ||
      overlap(y_fp16, yb, w->row_ptr, 4ull * (w->rows + 1)) ||
      (w->n_keep < 4 && overlap(y_fp16, yb, w->codes, (uint64_t)nnz / 4)))
    return fail(I4S_ERR_INVALID_ARGUMENT, "y overlaps a packed weight buffer");
  return I4S_OK;
}

}  // namespace

extern "C" {

i4s_status i4s_run(const i4s_packed *w, const uint16_t *x_fp16, int32_t batch, uint16_t *y_fp16,
                   void *stream) {
  i4s_status st = validate_run(w, x_fp16, batch, y_fp16);
  if (st != I4S_OK) return st;
  st = check_device();
  if (st != I4S_OK) return st;
  const hipError_t e = i4s::launch_gemv(*w, x_fp16, batch, y_fp16, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "gemv launch");
  return I4S_OK;
}

i4s_status i4s_run_workspace_size(const i4s_packed *w, int32_t batch, uint64_t *bytes) {
  if (!bytes) return fail(I4S_ERR_INVALID_ARGUMENT, "bytes is NULL");
  const i4s_status st = validate_layer(w, batch);
  if (st != I4S_OK) return st;
  *bytes = i4s::split_plan(*w, batch).workspace_bytes;
  return I4S_OK;
}

i4s_status i4s_run_ws(const i4s_packed *w, const uint16_t *x_fp16, int32_t batch, uint16_t *y_fp16,
                      void *workspace, uint64_t workspace_bytes, void *stream) {
  i4s_status st = validate_run(w, x_fp16, batch, y_fp16);
  if (st != I4S_OK) return st;
  const i4s::SplitPlan plan = i4s::split_plan(*w, batch);
  if (plan.workspace_bytes > 0) {
    if (!workspace || !aligned(workspace, 16))
      return fail(I4S_ERR_INVALID_ARGUMENT, "workspace is NULL or not 16-byte aligned");
    if (workspace_bytes < plan.workspace_bytes)
      return fail(I4S_ERR_WORKSPACE_TOO_SMALL, "workspace has %llu bytes, %llu needed",
                  (unsigned long long)workspace_bytes, (unsigned long long)plan.workspace_bytes);
    const uint64_t xb = 2ull * batch * w->cols, yb = 2ull * batch * w->rows;
    if (overlap(workspace, workspace_bytes, x_fp16, xb) || overlap(workspace, workspace_bytes, y_fp16, yb))
      return fail(I4S_ERR_INVALID_ARGUMENT, "workspace overlaps x or y");
  }
  st = check_device();
  if (st != I4S_OK) return st;
  const hipError_t e = i4s::launch_gemv_ws(*w, x_fp16, batch, y_fp16, plan, workspace,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "gemv launch");
  return I4S_OK;
}

i4s_status i4s_run_noalloc(const i4s_packed *w, const uint16_t *x_fp16, int32_t batch, uint16_t *y_fp16,
                           void *stream) {
  i4s_status st = validate_run(w, x_fp16, batch, y_fp16);
  if (st != I4S_OK) return st;
  const i4s::SplitPlan plan = i4s::split_plan(*w, batch);
  if (plan.workspace_bytes > I4S_NOALLOC_SCRATCH_BYTES)
    return fail(I4S_ERR_WORKSPACE_TOO_SMALL,
                "this layer and batch need %llu bytes of workspace, more than the %llu of the static scratch; "
                "use i4s_run_ws",
                (unsigned long long)plan.workspace_bytes, (unsigned long long)I4S_NOALLOC_SCRATCH_BYTES);
  st = check_device();
  if (st != I4S_OK) return st;
  void *ws = nullptr;
  if (plan.workspace_bytes > 0) {
    const hipError_t e = i4s::noalloc_scratch(&ws);
    if (e != hipSuccess) return device_error(e, "static scratch address");
  }
  const hipError_t e = i4s::launch_gemv_ws(*w, x_fp16, batch, y_fp16, plan, ws,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "gemv launch");
  return I4S_OK;
}

i4s_status i4s_run_multi(const i4s_packed *w, int32_t n, const uint16_t *x_fp16, int32_t batch,
                         uint16_t *const *y_fp16, void *stream) {
  if (!w || !y_fp16) return fail(I4S_ERR_INVALID_ARGUMENT, "w or y_fp16 is NULL");
  if (n < 1 || n > I4S_MAX_MULTI) return fail(I4S_ERR_INVALID_ARGUMENT, "n=%d must be in [1, %d]", n, I4S_MAX_MULTI);
  for (int32_t m = 0; m < n; ++m) {
    i4s_status st = validate_run(&w[m], x_fp16, batch, y_fp16[m]);
    if (st != I4S_OK) return st;
    if (w[m].cols != w[0].cols) return fail(I4S_ERR_INVALID_ARGUMENT, "layer %d has cols %d, layer 0 has %d", m,
                                            w[m].cols, w[0].cols);
  }
  // an output must not overlap another output or another layer's packed
  // buffers: in one launch all layers run at once
  for (int32_t m = 0; m < n; ++m) {
    const uint64_t yb = 2ull * batch * w[m].rows;
    for (int32_t j = 0; j < n; ++j) {
      if (j == m) continue;
      const i4s_packed &o = w[j];
      const int64_t nnz = o.nnz;
      if (overlap(y_fp16[m], yb, y_fp16[j], 2ull * batch * o.rows))
        return fail(I4S_ERR_INVALID_ARGUMENT, "outputs %d and %d overlap", m, j);
      if (overlap(y_fp16[m], yb, o.vals, (uint64_t)nnz / 2) ||
          overlap(y_fp16[m], yb, o.scales, 2ull * o.rows * (o.cols / o.group_size)) ||
          overlap(y_fp16[m], yb, o.row_ptr, 4ull * (o.rows + 1)) ||
          (o.n_keep < 4 && overlap(y_fp16[m], yb, o.codes, (uint64_t)nnz / 4)))
        return fail(I4S_ERR_INVALID_ARGUMENT, "output %d overlaps the packed buffers of layer %d", m, j);
    }
  }
  i4s_status st = check_device();
  if (st != I4S_OK) return st;
  const hipError_t e = i4s::launch_gemv_multi(w, n, x_fp16, batch, y_fp16, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "gemv launch");
  return I4S_OK;
}

const char *i4s_status_string(i4s_status s) {
  switch (s) {
    case I4S_OK: return "ok";
    case I4S_ERR_INVALID_ARGUMENT: return "invalid argument";
    case I4S_ERR_UNSUPPORTED: return "unsupported device";
    case I4S_ERR_NONFINITE_WEIGHT: return "non-finite weight";
    case I4S_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case I4S_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char *i4s_last_error(void) { return g_last_error.c_str(); }

int32_t i4s_version(void) { return 100; }

int32_t i4s_format_version(void) { return I4S_FORMAT_VERSION; }

}  // extern "C"
