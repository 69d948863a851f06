// Driver for the CPU build of libi4s's host layer (i4s_api.cpp, i4s_plan.cpp)
// against the HIP stand-in (i4s_hip_stub.cpp), built with AddressSanitizer
// and UndefinedBehaviorSanitizer.  Calls every entry point of include/i4s.h
// through its C ABI: the argument checks of each (every error comes back as
// the documented status before anything is launched), the adaptive group
// size decision on the SSE totals the analysis leaves behind, the K-split
// workspace plan, the rows kernel's launch shapes (every shape the plan can
// return has a kernel instantiation, fits the block size and the LDS), the
// no-allocation entry point's scratch limit, the device
// check (a device that reports another architecture gives
// I4S_ERR_UNSUPPORTED), and the status texts.  Prints "ok <n> checks" and
// exits 0 when every check holds.  Test infrastructure only.

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "i4s.h"
#include "i4s_hip_stub.h"
#include "i4s_internal.h"

namespace {

int g_checks = 0, g_fails = 0;

#define CHECK(cond)                                                                                      \
  do {                                                                                                   \
    ++g_checks;                                                                                          \
    if (!(cond)) {                                                                                       \
      ++g_fails;                                                                                         \
      std::fprintf(stderr, "%s:%d: CHECK(%s) failed; last error: %s\n", __FILE__, __LINE__, #cond,    \
                   i4s_last_error());                                                                    \
    }                                                                                                    \
  } while (0)
#define EXPECT(status, call) CHECK((call) == (status))

// "Device" buffers are host memory here, 256-byte aligned.
struct Buf {
  void *p = nullptr;
  explicit Buf(size_t n) { p = std::aligned_alloc(256, (n + 255) / 256 * 256 + 256); std::memset(p, 0, n); }
  ~Buf() { std::free(p); }
  template <typename T> T *as(size_t byte_offset = 0) const {
    return reinterpret_cast<T *>(static_cast<char *>(p) + byte_offset);
  }
};

// Addresses that are only compared and passed on, never dereferenced (the
// host layer never touches device memory).
template <typename T> T *fake(uint64_t gib) { return reinterpret_cast<T *>(static_cast<uintptr_t>(gib) << 30); }

void test_pack_sizes() {
  i4s_sizes s;
  EXPECT(I4S_OK, i4s_pack_sizes(4096, 4096, 2, 128, &s));
  CHECK(s.row_ptr == 4 * 4097ull && s.vals == 4194304ull && s.codes == 2097152ull && s.scales == 262144ull);
  CHECK(s.workspace > 0);
  EXPECT(I4S_OK, i4s_pack_sizes(64, 512, 4, 64, &s));
  CHECK(s.codes == 0 && s.vals == 64ull * 512 / 2 && s.scales == 2ull * 64 * 8);
  EXPECT(I4S_OK, i4s_pack_sizes(3, 768, 1, 0, &s));  // adaptive: scales sized for G = 64
  CHECK(s.scales == 2ull * 3 * 12 && s.codes == 3ull * 768 / 4 / 4);
  const int bad[][4] = {{0, 512, 2, 128},  {-1, 512, 2, 128}, {4, 0, 2, 128},  {4, 32, 2, 64},
                        {4, 100, 2, 64},   {4, 512, 3, 128},  {4, 512, 0, 128}, {4, 512, 2, 32},
                        {4, 512, 2, 512},  {4, 320, 2, 0},    {4, 320, 2, 128}, {65536, 32768, 4, 128},
                        {131072, 32768, 2, 128}};
  for (const auto &b : bad) EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack_sizes(b[0], b[1], b[2], b[3], &s));
  EXPECT(I4S_OK, i4s_pack_sizes(320, 320, 2, 64, &s));
  EXPECT(I4S_OK, i4s_pack_sizes(65535, 32768, 4, 128, &s));  // nnz just below 2^31
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack_sizes(4, 512, 2, 128, nullptr));
  CHECK(std::strlen(i4s_last_error()) > 0);
}

struct PackBufs {
  i4s_sizes s{};
  Buf *w, *rp, *vals, *codes, *scales, *ws;
  PackBufs(int rows, int cols, int n_keep, int g) {
    i4s_pack_sizes(rows, cols, n_keep, g, &s);
    w = new Buf(2ull * rows * cols);
    rp = new Buf(s.row_ptr);
    vals = new Buf(s.vals);
    codes = new Buf(s.codes + 16);
    scales = new Buf(s.scales);
    ws = new Buf(s.workspace);
  }
  ~PackBufs() { delete w; delete rp; delete vals; delete codes; delete scales; delete ws; }
  i4s_packed desc() const {
    i4s_packed d{};
    d.row_ptr = rp->as<int32_t>();
    d.vals = vals->as<uint8_t>();
    d.codes = codes->as<uint16_t>();
    d.scales = scales->as<uint16_t>();
    return d;
  }
};

int pack_with_totals(const uint64_t t[6], uint32_t flag, i4s_pack_report *rep) {
  i4s_stub_set_pack_result(flag, t);
  PackBufs b(32, 512, 2, 0);
  i4s_packed d = b.desc();
  return i4s_pack(b.w->as<uint16_t>(), 32, 512, 2, 0, b.ws->p, b.s.workspace, &d, rep, nullptr);
}

void test_pack() {
  i4s_pack_report rep;
  // the adaptive choice: smallest exact SSE, ties to the larger group (lo, hi per candidate)
  const uint64_t tie_64_128[6] = {5, 0, 5, 0, 7, 0};
  EXPECT(I4S_OK, pack_with_totals(tie_64_128, 0, &rep));
  CHECK(rep.group_size == 128 && rep.n_candidates == 3 && rep.candidates[0] == 64 && rep.candidates[2] == 256);
  CHECK(rep.sse_lo[0] == 5 && rep.sse_lo[2] == 7 && rep.sse_hi[1] == 0);
  CHECK(i4s_stub_last_launch().kind == 2 && i4s_stub_last_launch().group_size == 128);
  const uint64_t smallest_64[6] = {3, 0, 5, 0, 7, 0};
  EXPECT(I4S_OK, pack_with_totals(smallest_64, 0, &rep));
  CHECK(rep.group_size == 64);
  const uint64_t all_equal[6] = {7, 0, 7, 0, 7, 0};
  EXPECT(I4S_OK, pack_with_totals(all_equal, 0, &rep));
  CHECK(rep.group_size == 256);
  const uint64_t high_words[6] = {0, 2, ~0ull, 1, 0, 3};  // 128-bit compare: the high word decides
  EXPECT(I4S_OK, pack_with_totals(high_words, 0, &rep));
  CHECK(rep.group_size == 128 && rep.sse_hi[1] == 1 && rep.sse_lo[1] == ~0ull);
  // flags raised by the analysis
  EXPECT(I4S_ERR_NONFINITE_WEIGHT, pack_with_totals(all_equal, 1, &rep));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, pack_with_totals(all_equal, 2, &rep));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, pack_with_totals(all_equal, 4, &rep));
  EXPECT(I4S_ERR_NONFINITE_WEIGHT, pack_with_totals(all_equal, 7, &rep));  // a bad weight is reported first
  const uint64_t zero[6] = {};
  i4s_stub_set_pack_result(0, zero);

  PackBufs b(32, 512, 2, 128);
  i4s_packed d = b.desc();
  uint16_t *w = b.w->as<uint16_t>();
  EXPECT(I4S_OK, i4s_pack(w, 32, 512, 2, 128, b.ws->p, b.s.workspace, &d, &rep, nullptr));
  CHECK(rep.group_size == 128 && rep.n_candidates == 0 && d.group_size == 128 && d.nnz == 32 * 512 / 2);
  CHECK(d.rows == 32 && d.cols == 512 && d.n_keep == 2);
  EXPECT(I4S_OK, i4s_pack(w, 32, 512, 2, 128, b.ws->p, b.s.workspace, &d, nullptr, nullptr));
  // argument checks: nothing is launched
  const int before = i4s_stub_launches();
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack(nullptr, 32, 512, 2, 128, b.ws->p, b.s.workspace, &d, &rep, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack(w + 1, 32, 512, 2, 128, b.ws->p, b.s.workspace, &d, &rep, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack(w, 32, 512, 2, 128, b.ws->p, b.s.workspace, nullptr, &rep, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack(w, 32, 512, 3, 128, b.ws->p, b.s.workspace, &d, &rep, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack(w, 32, 512, 2, 128, nullptr, b.s.workspace, &d, &rep, nullptr));
  EXPECT(I4S_ERR_WORKSPACE_TOO_SMALL, i4s_pack(w, 32, 512, 2, 128, b.ws->p, b.s.workspace - 1, &d, &rep, nullptr));
  i4s_packed e = d;
  e.codes = nullptr;
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack(w, 32, 512, 2, 128, b.ws->p, b.s.workspace, &e, &rep, nullptr));
  e = d;
  e.vals = b.vals->as<uint8_t>(8);  // misaligned
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack(w, 32, 512, 2, 128, b.ws->p, b.s.workspace, &e, &rep, nullptr));
  e = d;
  e.scales = reinterpret_cast<uint16_t *>(d.vals);  // outputs overlap
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack(w, 32, 512, 2, 128, b.ws->p, b.s.workspace, &e, &rep, nullptr));
  e = d;
  e.row_ptr = reinterpret_cast<int32_t *>(w);  // an output overlaps W
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack(w, 32, 512, 2, 128, b.ws->p, b.s.workspace, &e, &rep, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack(w, 32, 512, 2, 128, d.vals, b.s.workspace, &d, &rep, nullptr));
  Buf norms(4 * 512 + 16);
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack_ex(w, 32, 512, 2, 128, norms.as<float>(4), nullptr, b.ws->p,
                                               b.s.workspace, &d, &rep, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_pack_ex(w, 32, 512, 2, 128, nullptr, w + 4, b.ws->p, b.s.workspace, &d,
                                               &rep, nullptr));
  CHECK(i4s_stub_launches() == before);
  EXPECT(I4S_OK, i4s_pack_ex(w, 32, 512, 2, 128, norms.as<float>(), nullptr, b.ws->p, b.s.workspace, &d, &rep,
                             nullptr));
  // dense: codes may be NULL
  PackBufs dn(8, 256, 4, 64);
  i4s_packed dd = dn.desc();
  dd.codes = nullptr;
  EXPECT(I4S_OK, i4s_pack(dn.w->as<uint16_t>(), 8, 256, 4, 64, dn.ws->p, dn.s.workspace, &dd, &rep, nullptr));
  CHECK(dd.codes == nullptr);
}

// A packed layer's descriptor over fresh buffers.
struct Layer {
  int rows, cols, n_keep, g;
  Buf *rp, *vals, *codes, *scales;
  Layer(int r, int c, int n, int gs) : rows(r), cols(c), n_keep(n), g(gs) {
    i4s_sizes s;
    i4s_pack_sizes(r, c, n, gs, &s);
    rp = new Buf(s.row_ptr);
    vals = new Buf(s.vals);
    codes = new Buf(s.codes + 16);
    scales = new Buf(s.scales);
  }
  ~Layer() { delete rp; delete vals; delete codes; delete scales; }
  i4s_packed desc() const {
    i4s_packed d{};
    d.rows = rows; d.cols = cols; d.n_keep = n_keep; d.group_size = g;
    d.nnz = (int64_t)rows * cols / 4 * n_keep;
    d.row_ptr = rp->as<int32_t>(); d.vals = vals->as<uint8_t>();
    d.codes = n_keep < 4 ? codes->as<uint16_t>() : nullptr; d.scales = scales->as<uint16_t>();
    return d;
  }
};

void test_run() {
  Layer L(64, 1024, 2, 128);
  const i4s_packed d = L.desc();
  Buf x(2 * 16 * 1024 + 64), y(2 * 16 * 64 + 64);
  uint16_t *xp = x.as<uint16_t>(), *yp = y.as<uint16_t>();
  for (int b = 1; b <= 16; ++b) {
    EXPECT(I4S_OK, i4s_run(&d, xp, b, yp, nullptr));
    CHECK(i4s_stub_last_launch().kind == 3 && i4s_stub_last_launch().batch == b);
  }
  const int before = i4s_stub_launches();
  i4s_packed e = d;
  e.nnz += 1;
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&e, xp, 1, yp, nullptr));
  for (int gs : {0, 32, 512, 96}) {
    e = d;
    e.group_size = gs;
    EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&e, xp, 1, yp, nullptr));
  }
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&d, xp, 0, yp, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&d, xp, 17, yp, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(nullptr, xp, 1, yp, nullptr));
  e = d; e.vals = nullptr;
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&e, xp, 1, yp, nullptr));
  e = d; e.vals = L.vals->as<uint8_t>(8);
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&e, xp, 1, yp, nullptr));
  e = d; e.codes = L.codes->as<uint16_t>(4);
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&e, xp, 1, yp, nullptr));
  e = d; e.codes = nullptr;
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&e, xp, 1, yp, nullptr));
  e = d; e.row_ptr = L.rp->as<int32_t>(2);
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&e, xp, 1, yp, nullptr));
  e = d; e.scales = L.scales->as<uint16_t>(1);
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&e, xp, 1, yp, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&d, xp + 1, 1, yp, nullptr));      // x misaligned
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&d, xp, 1, y.as<uint16_t>(1), nullptr));  // y misaligned
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&d, xp, 1, nullptr, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&d, xp, 2, xp + 1024, nullptr));   // y inside x
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&d, xp, 1, reinterpret_cast<uint16_t *>(d.vals), nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&d, xp, 1, d.scales, nullptr));
  CHECK(i4s_stub_launches() == before);
  Layer D(16, 512, 4, 64);  // dense: no codes
  const i4s_packed dd = D.desc();
  EXPECT(I4S_OK, i4s_run(&dd, xp, 3, yp, nullptr));
}

// A process whose device is another architecture: every entry point that
// would touch the device returns I4S_ERR_UNSUPPORTED and launches nothing;
// the host-only ones still answer.  (The library remembers the answer per
// device, so this runs in a process of its own.)
void test_other_architecture(const char *arch) {
  i4s_stub_set_arch(arch);
  PackBufs b(32, 512, 2, 128);
  i4s_packed pd = b.desc();
  i4s_pack_report rep;
  uint16_t *w = b.w->as<uint16_t>();
  Layer L(256, 40960, 2, 128);
  const i4s_packed d = L.desc();
  Buf x(2 * 4 * 40960 + 64), y(2 * 4 * 256 + 64), ws(16 << 20);
  uint16_t *xp = x.as<uint16_t>(), *yp = y.as<uint16_t>();
  uint16_t *ys[1] = {yp};
  EXPECT(I4S_ERR_UNSUPPORTED, i4s_pack(w, 32, 512, 2, 128, b.ws->p, b.s.workspace, &pd, &rep, nullptr));
  CHECK(std::strstr(i4s_last_error(), arch) != nullptr);  // the first check names the architecture
  EXPECT(I4S_ERR_UNSUPPORTED, i4s_pack_ex(w, 32, 512, 2, 0, nullptr, nullptr, b.ws->p, b.s.workspace, &pd, &rep,
                                          nullptr));
  EXPECT(I4S_ERR_UNSUPPORTED, i4s_run(&d, xp, 1, yp, nullptr));
  EXPECT(I4S_ERR_UNSUPPORTED, i4s_run_ws(&d, xp, 4, yp, ws.p, 16 << 20, nullptr));
  EXPECT(I4S_ERR_UNSUPPORTED, i4s_run_noalloc(&d, xp, 4, yp, nullptr));
  EXPECT(I4S_ERR_UNSUPPORTED, i4s_run_multi(&d, 1, xp, 4, ys, nullptr));
  CHECK(i4s_stub_launches() == 0);
  // argument errors are still reported as such (they are checked first)
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run(&d, xp, 0, yp, nullptr));
  i4s_sizes s;
  uint64_t n = 0;
  EXPECT(I4S_OK, i4s_pack_sizes(32, 512, 2, 0, &s));
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 4, &n));
  CHECK(n > 0);
}

void test_workspace_and_noalloc() {
  uint64_t n = 1;
  // batch 1, other patterns and short rows need no workspace
  i4s_packed d{};
  d.rows = 4096; d.cols = 40960; d.n_keep = 2; d.group_size = 128; d.nnz = 4096ll * 40960 / 2;
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 1, &n));
  CHECK(n == 0);
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 4, &n));
  CHECK(n > 0 && n % 1024 == 0 && n <= I4S_NOALLOC_SCRATCH_BYTES);
  d.n_keep = 1; d.nnz = 4096ll * 40960 / 4;
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 4, &n));
  CHECK(n == 0);
  d.n_keep = 2; d.cols = 20480; d.nnz = 4096ll * 20480 / 2;
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 16, &n));
  CHECK(n > 0);  // batch > 8, K >= 5120 on at most 512 tiles
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 8, &n));
  CHECK(n > 0);  // batch 8 on 4096 rows: the rows kernel's 256 blocks
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 4, &n));
  CHECK(n == 0);  // ... but not below batch 8
  d.rows = 5000; d.nnz = 5000ll * 20480 / 2;
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 16, &n));
  CHECK(n > 0);  // 313 tiles
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 8, &n));
  CHECK(n > 0);  // batch <= 8, the rows kernel's 157 blocks
  d.rows = 9000; d.nnz = 9000ll * 20480 / 2;
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 16, &n));
  CHECK(n == 0);  // 563 tiles: a tall layer keeps the rows kernel
  d.rows = 5000; d.cols = 4096; d.nnz = 5000ll * 4096 / 2;
  EXPECT(I4S_OK, i4s_run_workspace_size(&d, 16, &n));
  CHECK(n == 0);  // K < 5120
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_workspace_size(&d, 16, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_workspace_size(&d, 0, &n));

  // a layer that splits K: 256 x 40960, 2:4
  Layer L(256, 40960, 2, 128);
  const i4s_packed s = L.desc();
  Buf x(2 * 16 * 40960 + 64), y(2 * 16 * 256 + 64);
  uint16_t *xp = x.as<uint16_t>(), *yp = y.as<uint16_t>();
  EXPECT(I4S_OK, i4s_run_workspace_size(&s, 4, &n));
  CHECK(n > 0);
  Buf ws(n);
  const int before = i4s_stub_launches();
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_ws(&s, xp, 4, yp, nullptr, n, nullptr));
  EXPECT(I4S_ERR_WORKSPACE_TOO_SMALL, i4s_run_ws(&s, xp, 4, yp, ws.p, n - 1, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_ws(&s, xp, 4, yp, ws.as<char>(8), n, nullptr));  // misaligned
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_ws(&s, xp, 4, yp, xp, n, nullptr));             // overlaps x
  CHECK(i4s_stub_launches() == before);
  EXPECT(I4S_OK, i4s_run_ws(&s, xp, 4, yp, ws.p, n, nullptr));
  CHECK(i4s_stub_last_launch().kind == 4 && i4s_stub_last_launch().workspace == ws.p);
  EXPECT(I4S_OK, i4s_run_ws(&s, xp, 1, yp, nullptr, 0, nullptr));  // batch 1: no workspace needed
  // the no-allocation entry point hands the static scratch to the split
  EXPECT(I4S_OK, i4s_run_noalloc(&s, xp, 4, yp, nullptr));
  CHECK(i4s_stub_last_launch().kind == 4 && i4s_stub_last_launch().workspace == i4s_stub_scratch());
  EXPECT(I4S_OK, i4s_run_noalloc(&s, xp, 1, yp, nullptr));
  CHECK(i4s_stub_last_launch().workspace == nullptr);
  // ... and refuses a split beyond its array before anything is launched
  i4s_packed big{};
  big.rows = 16384; big.cols = 65536; big.n_keep = 2; big.group_size = 128; big.nnz = 16384ll * 65536 / 2;
  EXPECT(I4S_OK, i4s_run_workspace_size(&big, 16, &n));
  CHECK(n > I4S_NOALLOC_SCRATCH_BYTES);
  big.row_ptr = fake<int32_t>(1); big.vals = fake<uint8_t>(2); big.codes = fake<uint16_t>(4);
  big.scales = fake<uint16_t>(6);
  const int b2 = i4s_stub_launches();
  EXPECT(I4S_ERR_WORKSPACE_TOO_SMALL, i4s_run_noalloc(&big, fake<uint16_t>(8), 16, fake<uint16_t>(9), nullptr));
  CHECK(i4s_stub_launches() == b2);
  CHECK(std::strstr(i4s_last_error(), "i4s_run_ws") != nullptr);
}

void test_multi() {
  Layer a(40, 512, 2, 64), b(70, 512, 2, 64), c(40, 1024, 2, 64);
  const i4s_packed ds[3] = {a.desc(), b.desc(), c.desc()};
  Buf x(2 * 4 * 1024 + 64), y0(2 * 4 * 40), y1(2 * 4 * 70);
  uint16_t *xp = x.as<uint16_t>();
  uint16_t *ys[2] = {y0.as<uint16_t>(), y1.as<uint16_t>()};
  EXPECT(I4S_OK, i4s_run_multi(ds, 2, xp, 4, ys, nullptr));
  CHECK(i4s_stub_last_launch().kind == 5 && i4s_stub_last_launch().layers == 2);
  const int before = i4s_stub_launches();
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_multi(ds, 0, xp, 4, ys, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_multi(ds, I4S_MAX_MULTI + 1, xp, 4, ys, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_multi(nullptr, 2, xp, 4, ys, nullptr));
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_multi(ds, 2, xp, 4, nullptr, nullptr));
  const i4s_packed mixed[2] = {a.desc(), c.desc()};  // different cols
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_multi(mixed, 2, xp, 4, ys, nullptr));
  uint16_t *same[2] = {y1.as<uint16_t>(), y1.as<uint16_t>()};  // outputs overlap
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_multi(ds, 2, xp, 4, same, nullptr));
  uint16_t *into_b[2] = {reinterpret_cast<uint16_t *>(ds[1].vals), y1.as<uint16_t>()};  // output 0 inside layer 1
  EXPECT(I4S_ERR_INVALID_ARGUMENT, i4s_run_multi(ds, 2, xp, 4, into_b, nullptr));
  CHECK(i4s_stub_launches() == before);
}

// rows_shape over every K the rows kernel takes (up to 512 units), tile
// counts around each of its thresholds, batch 2..16 and N = 1, 2, 4: the
// (chunk width, chunks per wave, tiles per wave) triple is one of the
// instantiated kernels, the waves cover the chunks exactly once, the block
// fits the kernel's work-group limit, the LDS is what the kernel addresses
// and fits 160 KB, and the compact B fragments (bv 4 / 8 / 16 at batch <=
// 4 / <= 8 / above) are chosen only in the shapes instantiated for them
// (1:4 at batch <= 8 only with one 8-unit chunk per wave, 16 only with one
// tile per wave or four 2:4 tiles) and only where they leave as many blocks per CU
// or the blocks fit the 256 CUs once.
void test_rows_shapes() {
  const int tiles_set[] = {1, 2, 7, 16, 100, 159, 160, 161, 255, 256, 257, 299, 300, 301, 320,
                           511, 512, 513, 639, 640, 641, 700, 864, 1000, 2000, 5000};
  long bad = 0;
  char first[160] = "";
  for (int nk : {1, 2, 4})
    for (int units = 1; units <= 512; ++units)
      for (int t : tiles_set)
        for (int b = 2; b <= 16; ++b) {
          const i4s::RowsShape r = i4s::rows_shape(units, t, b, nk);
          const bool inst =
              (r.u == 16 && ((r.cpw == 1 && (r.tpw == 1 || r.tpw == 2)) ||
                             (r.cpw == 2 && (r.tpw == 1 || (r.tpw == 2 && nk != 4))) || (r.cpw == 4 && r.tpw == 1))) ||
              (r.u == 8 && r.cpw == 1 && (r.tpw == 1 || r.tpw == 2 || (r.tpw == 4 && nk == 2)));
          const int chunks = inst ? (units + r.u - 1) / r.u : 0;
          const int maxw = r.tpw == 4 ? 12 : (r.u == 8 ? 16 : 8);
          // the LDS is the waves' tile areas plus, with compact B fragments,
          // the activations' area
          const size_t tile = nk == 4 ? (r.u == 8 ? i4s::RowsGeom<8, 4>::kTileLds : i4s::RowsGeom<16, 4>::kTileLds)
                              : nk == 1 ? (r.u == 8 ? i4s::RowsGeom<8, 1>::kTileLds : i4s::RowsGeom<16, 1>::kTileLds)
                                        : (r.u == 8 ? i4s::RowsGeom<8>::kTileLds : i4s::RowsGeom<16>::kTileLds);
          const size_t base = (size_t)r.waves * r.tpw * tile;
          const bool compact_shape = r.bv == 16 ? (b > 8 && (r.tpw == 1 || (r.tpw == 4 && nk == 2)))
                                   : (r.bv == 8 ? b > 4 && b <= 8 : b <= 4) && r.tpw <= 2 &&
                                         (nk != 1 || (r.u == 8 && r.cpw == 1));
          const bool bv_ok = (r.bv == 0 && r.lds == base) ||
                             ((r.bv == 4 || r.bv == 8 || r.bv == 16) && compact_shape &&
                              r.lds == base + (size_t)r.waves * i4s::kRowsBcBytes &&
                              ((160 * 1024) / r.lds == (160 * 1024) / base || (t + r.tpw - 1) / r.tpw <= 256));
          const bool ok = inst && bv_ok && r.waves >= 1 && r.waves * r.cpw >= chunks &&
                          (r.waves - 1) * r.cpw < chunks && r.waves <= maxw && r.lds > 0 && r.lds <= 160 * 1024;
          if (!ok && bad++ == 0)
            std::snprintf(first, sizeof first,
                          "units %d tiles %d batch %d N %d -> u %d cpw %d tpw %d waves %d bv %d lds %zu", units, t, b,
                          nk, r.u, r.cpw, r.tpw, r.waves, r.bv, r.lds);
        }
  if (bad) std::fprintf(stderr, "rows_shape: %ld bad shapes, first: %s\n", bad, first);
  CHECK(bad == 0);
}

void test_status() {
  const i4s_status all[] = {I4S_OK, I4S_ERR_INVALID_ARGUMENT, I4S_ERR_UNSUPPORTED, I4S_ERR_NONFINITE_WEIGHT,
                            I4S_ERR_WORKSPACE_TOO_SMALL, I4S_ERR_DEVICE};
  for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) {
    CHECK(i4s_status_string(all[i]) != nullptr && std::strlen(i4s_status_string(all[i])) > 0);
    for (size_t j = 0; j < i; ++j) CHECK(std::strcmp(i4s_status_string(all[i]), i4s_status_string(all[j])) != 0);
  }
  CHECK(std::strcmp(i4s_status_string(static_cast<i4s_status>(99)), "unknown status") == 0);
  CHECK(i4s_version() == 100 && i4s_format_version() == I4S_FORMAT_VERSION);
}

}  // namespace

int main(int argc, char **argv) {
  if (argc > 2 && std::strcmp(argv[1], "--arch") == 0) {
    test_other_architecture(argv[2]);
  } else {
    test_pack_sizes();
    test_pack();
    test_run();
    test_workspace_and_noalloc();
    test_multi();
    test_rows_shapes();
    test_status();
  }
  if (g_fails) {
    std::printf("FAILED %d of %d checks\n", g_fails, g_checks);
    return 1;
  }
  std::printf("ok %d checks\n", g_checks);
  return 0;
}
