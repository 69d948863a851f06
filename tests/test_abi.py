"""CPU tests of the C ABI: the library loads, exports every declared symbol,
its structs match the header's layout, and host-side validation returns the
documented status before touching a device.  No compute call runs here."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from int4_sparse_gemv_amd import _binding as B
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "i4s.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from int4_sparse_gemv_amd import build
        build.build()
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(i4s_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(
        ["i4s_pack_sizes", "i4s_pack", "i4s_pack_ex", "i4s_run", "i4s_run_workspace_size", "i4s_run_ws",
         "i4s_run_multi", "i4s_run_noalloc",
         "i4s_status_string", "i4s_last_error", "i4s_version", "i4s_format_version"])


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (i4s_[a-z_]+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(B.SIGNATURES) == set(declared_functions())


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "i4s.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu\n", sizeof(i4s_packed), offsetof(i4s_packed, nnz),
         offsetof(i4s_packed, row_ptr), offsetof(i4s_packed, codes), offsetof(i4s_packed, scales));
  printf("%zu %zu\n", sizeof(i4s_sizes), offsetof(i4s_sizes, workspace));
  printf("%zu %zu %zu\n", sizeof(i4s_pack_report), offsetof(i4s_pack_report, sse_hi),
         offsetof(i4s_pack_report, sse_lo));
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    P, S, R = B.i4s_packed, B.i4s_sizes, B.i4s_pack_report
    assert lines[0].split() == [str(v) for v in (ctypes.sizeof(P), P.nnz.offset, P.row_ptr.offset,
                                                 P.codes.offset, P.scales.offset)]
    assert lines[1].split() == [str(v) for v in (ctypes.sizeof(S), S.workspace.offset)]
    assert lines[2].split() == [str(v) for v in (ctypes.sizeof(R), R.sse_hi.offset, R.sse_lo.offset)]


def test_version_and_status_strings(lib):
    assert B.i4s_version() >= 100
    assert B.i4s_format_version() == B.I4S_FORMAT_VERSION == 1
    for st in range(6):
        assert B.i4s_status_string(st)
    assert B.i4s_status_string(99) == "unknown status"


@pytest.mark.parametrize("rows,cols,n_keep,g", [
    (512, 512, 2, 128), (4096, 4096, 2, 128), (11008, 4096, 2, 0), (4096, 11008, 2, 64),
    (4096, 4096, 4, 64), (13824, 5120, 2, 128), (3, 192, 1, 64), (1, 64, 4, 64),
    (65535, 32768, 4, 128), (131071, 32768, 2, 128)])   # nnz just below 2**31
def test_pack_sizes_match_closed_form(lib, rows, cols, n_keep, g):
    sz = B.i4s_sizes()
    assert B.i4s_pack_sizes(rows, cols, n_keep, g, sz) == B.I4S_OK
    want = oracle.packed_nbytes(rows, cols, n_keep, g or 64)
    assert (sz.row_ptr, sz.vals, sz.codes, sz.scales) == (want["row_ptr"], want["vals"], want["codes"],
                                                          want["scales"])
    assert sz.workspace >= 64


@pytest.mark.parametrize("rows,cols,n_keep,g", [
    (0, 512, 2, 128), (4, 96, 2, 64), (4, 512, 3, 128), (4, 512, 2, 32), (4, 192, 2, 128),
    (4, 320, 2, 0), (4, 576, 2, 256), (1 << 20, 1 << 12, 4, 64), (-1, 64, 2, 64),
    (65536, 32768, 4, 128), (131072, 32768, 2, 128)])   # nnz = 2**31
def test_pack_sizes_rejects(lib, rows, cols, n_keep, g):
    sz = B.i4s_sizes()
    assert B.i4s_pack_sizes(rows, cols, n_keep, g, sz) == B.I4S_ERR_INVALID_ARGUMENT
    assert B.i4s_last_error()


def test_pack_sizes_null_out(lib):
    assert lib.i4s_pack_sizes(64, 64, 2, 64, None) == B.I4S_ERR_INVALID_ARGUMENT


def _desc(rows=64, cols=256, n_keep=2, g=128, base=1 << 20):
    d = B.i4s_packed()
    d.rows, d.cols, d.n_keep, d.group_size = rows, cols, n_keep, g
    d.nnz = rows * cols * n_keep // 4
    d.row_ptr, d.vals, d.codes, d.scales = base, base + (1 << 16), base + (2 << 16), base + (3 << 16)
    return d


@pytest.mark.parametrize("mutate,batch", [
    (lambda d: setattr(d, "group_size", 0), 1),
    (lambda d: setattr(d, "group_size", 96), 1),
    (lambda d: setattr(d, "nnz", 5), 1),
    (lambda d: setattr(d, "vals", (1 << 20) + 8), 1),
    (lambda d: setattr(d, "codes", None), 1),
    (lambda d: setattr(d, "n_keep", 3), 1),
    (lambda d: None, 0),
    (lambda d: None, 17),
])
def test_run_validation_fails_before_any_device_call(lib, mutate, batch):
    d = _desc()
    mutate(d)
    x, y = 1 << 30, 1 << 31
    assert B.i4s_run(d, x, batch, y, None) == B.I4S_ERR_INVALID_ARGUMENT
    assert B.i4s_last_error()


def test_run_rejects_overlap_and_misalignment(lib):
    d = _desc()
    assert B.i4s_run(d, 1 << 30, 1, (1 << 30) + 64, None) == B.I4S_ERR_INVALID_ARGUMENT  # x/y overlap
    assert B.i4s_run(d, (1 << 30) + 2, 1, 1 << 31, None) == B.I4S_ERR_INVALID_ARGUMENT   # x misaligned
    assert B.i4s_run(d, 1 << 30, 1, (1 << 20) + (1 << 16), None) == B.I4S_ERR_INVALID_ARGUMENT  # y on vals
    assert lib.i4s_run(None, 1 << 30, 1, 1 << 31, None) == B.I4S_ERR_INVALID_ARGUMENT


def test_run_multi_validation_fails_before_any_device_call(lib):
    x = 1 << 30
    a, b = _desc(base=1 << 20), _desc(base=1 << 24)
    y0, y1 = 1 << 31, (1 << 31) + (1 << 20)
    E = B.I4S_ERR_INVALID_ARGUMENT
    assert B.i4s_run_multi([], x, 1, [], None) == E                         # n = 0
    assert B.i4s_run_multi([a] * 9, x, 1, [y0 + (k << 20) for k in range(9)], None) == E  # n > 8
    assert lib.i4s_run_multi(None, 1, x, 1, None, None) == E
    c = _desc(cols=512, base=1 << 24)
    assert B.i4s_run_multi([a, c], x, 1, [y0, y1], None) == E               # cols differ
    assert B.i4s_run_multi([a, b], x, 1, [y0, y0 + 64], None) == E          # outputs overlap
    assert B.i4s_run_multi([a, b], x, 1, [y0, (1 << 20) + (1 << 16)], None) == E  # y1 on layer 0's vals
    assert B.i4s_run_multi([a, b], x, 17, [y0, y1], None) == E              # batch out of range
    bad = _desc(base=1 << 24)
    bad.nnz = 5
    assert B.i4s_run_multi([a, bad], x, 1, [y0, y1], None) == E             # a bad descriptor
    assert "layer" in B.i4s_last_error() or B.i4s_last_error()


def test_pack_validation_fails_before_any_device_call(lib):
    sz = B.i4s_sizes()
    assert B.i4s_pack_sizes(64, 256, 2, 0, sz) == B.I4S_OK
    d = _desc()
    rep = B.i4s_pack_report()
    w, ws = 1 << 30, 1 << 31
    # workspace too small
    assert B.i4s_pack(w, 64, 256, 2, 0, ws, sz.workspace - 1, d, rep, None) == B.I4S_ERR_WORKSPACE_TOO_SMALL
    # misaligned weight, null workspace, bad shape
    assert B.i4s_pack(w + 2, 64, 256, 2, 0, ws, sz.workspace, d, rep, None) == B.I4S_ERR_INVALID_ARGUMENT
    assert B.i4s_pack(w, 64, 256, 2, 0, None, sz.workspace, d, rep, None) == B.I4S_ERR_INVALID_ARGUMENT
    assert B.i4s_pack(w, 64, 250, 2, 0, ws, sz.workspace, d, rep, None) == B.I4S_ERR_INVALID_ARGUMENT
    d.codes = None
    assert B.i4s_pack(w, 64, 256, 2, 0, ws, sz.workspace, d, rep, None) == B.I4S_ERR_INVALID_ARGUMENT
    # i4s_pack_ex: misaligned importance inputs are rejected on the host
    d = _desc()
    n, g = 1 << 32, 1 << 33
    assert B.i4s_pack_ex(w, 64, 256, 2, 0, n + 4, None, ws, sz.workspace, d, rep, None) == B.I4S_ERR_INVALID_ARGUMENT
    assert B.i4s_pack_ex(w, 64, 256, 2, 0, None, g + 2, ws, sz.workspace, d, rep, None) == B.I4S_ERR_INVALID_ARGUMENT
    assert B.i4s_pack_ex(w, 64, 256, 2, 0, n, g, ws, sz.workspace - 1, d, rep, None) == B.I4S_ERR_WORKSPACE_TOO_SMALL
    assert B.i4s_pack_ex(w, 64, 250, 2, 0, n, g, ws, sz.workspace, d, rep, None) == B.I4S_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("case", ["ws_on_w", "vals_on_w", "codes_on_scales", "row_ptr_on_ws", "scales_on_grad",
                                  "vals_on_norm"])
def test_pack_rejects_overlapping_buffers(lib, case):
    sz = B.i4s_sizes()
    assert B.i4s_pack_sizes(64, 256, 2, 0, sz) == B.I4S_OK
    d = _desc()
    w, ws, n, g = 1 << 30, 1 << 31, 1 << 32, 1 << 33
    if case == "ws_on_w":
        ws = w + 2 * 64 * 256 - 16
    elif case == "vals_on_w":
        d.vals = w + 1024
    elif case == "codes_on_scales":
        d.codes = d.scales + sz.scales - 16
    elif case == "row_ptr_on_ws":
        d.row_ptr = ws + sz.workspace - 16
    elif case == "scales_on_grad":
        d.scales = g + 4096
    else:
        d.vals = n
    st = B.i4s_pack_ex(w, 64, 256, 2, 0, n, g, ws, sz.workspace, d, None, None)
    assert st == B.I4S_ERR_INVALID_ARGUMENT
    assert "overlap" in B.i4s_last_error()


def test_binding_without_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError):
        B._lib_saved = B._lib
        try:
            B._lib = None
            B.load(str(tmp_path / "missing.so"))
        finally:
            B._lib = B._lib_saved


def _split_workspace(rows, cols):
    """Bytes of the K split's fp32 partial tiles: slices of 16 units (1024
    columns) x groups of 4 waves x tw 16-row tiles, 64 lanes x 16 bytes per
    tile; tw = 2 where that still leaves >= 384 blocks."""
    units, tiles = cols // 64, -(-rows // 16)
    ksplit = -(-units // 16)
    tw = 2 if ksplit * -(-tiles // 8) >= 384 else 1
    return ksplit * -(-tiles // (4 * tw)) * 4 * tw * 64 * 16 if ksplit > 1 else 0


def test_run_workspace_size_is_host_only_and_planned(lib):
    n = ctypes.c_uint64()

    def size(rows, cols, batch, n_keep=2, g=128):
        assert B.i4s_run_workspace_size(_desc(rows, cols, n_keep, g), batch, n) == B.I4S_OK
        return n.value
    # batch 1 and non-2:4 patterns need no workspace
    assert size(4096, 4096, 1) == 0 and size(4096, 4096, 8, n_keep=4) == 0 and size(4096, 4096, 8, n_keep=1) == 0
    # tall layers and short rows run the one-launch rows kernel at every batch
    for batch in (2, 3, 4, 8, 16):
        assert size(13824, 5120, batch) == 0 and size(14336, 4096, batch) == 0 and size(4096, 4096, batch) == 0
    # batch 2 never splits below K = 32768
    assert size(5120, 13824, 2) == 0 and size(1024, 16384, 2) == 0
    # batch 3-8: long rows (K >= 8192) on layers where the rows kernel would
    # run fewer than 192 blocks split K; 4096 rows (256 blocks) only at batch 8
    for batch in (3, 4, 8):
        assert size(5120, 13824, batch) == _split_workspace(5120, 13824) == 4587520
        assert size(2048, 8192, batch) == _split_workspace(2048, 8192) > 0
        assert size(5120, 5120, batch) == 0
    for batch in (3, 4, 7):
        assert size(4096, 11008, batch) == 0 and size(8208, 8192, batch) == 0
    assert size(4096, 11008, 8) == _split_workspace(4096, 11008) > 0
    assert size(8208, 8192, 8) == 0  # 257 blocks
    # batch 9-16: K >= 5120 on at most 512 tiles
    for batch in (9, 16):
        for rows, cols in ((5120, 5120), (4096, 11008), (8192, 8192), (4096, 28672)):
            assert size(rows, cols, batch) == _split_workspace(rows, cols) > 0
        assert size(8208, 8192, batch) == 0  # 513 tiles
    # beyond K = 32768 the rows kernel does not fit: every batch >= 2 splits
    for batch in (2, 4, 16):
        assert size(5120, 40960, batch) == _split_workspace(5120, 40960) > 0
    # a single slice (K <= 1024) needs no partials
    assert size(64, 1024, 16) == 0
    assert B.i4s_run_workspace_size(_desc(), 0, n) == B.I4S_ERR_INVALID_ARGUMENT
    assert lib.i4s_run_workspace_size(ctypes.byref(_desc()), 2, None) == B.I4S_ERR_INVALID_ARGUMENT


def test_run_ws_validation_fails_before_any_device_call(lib):
    d = _desc(4096, 20480, 2, 128)
    n = ctypes.c_uint64()
    assert B.i4s_run_workspace_size(d, 16, n) == B.I4S_OK
    x, y, ws = 1 << 34, 1 << 35, 1 << 36
    assert B.i4s_run_ws(d, x, 16, y, ws, n.value - 1, None) == B.I4S_ERR_WORKSPACE_TOO_SMALL
    assert B.i4s_run_ws(d, x, 16, y, None, n.value, None) == B.I4S_ERR_INVALID_ARGUMENT
    assert B.i4s_run_ws(d, x, 16, y, ws + 8, n.value, None) == B.I4S_ERR_INVALID_ARGUMENT
    assert B.i4s_run_ws(d, x, 16, y, x, n.value, None) == B.I4S_ERR_INVALID_ARGUMENT  # overlaps x
    assert B.i4s_run_ws(d, x, 17, y, ws, n.value, None) == B.I4S_ERR_INVALID_ARGUMENT


def test_floor_library_exports_and_rejects_bad_arguments():
    """The benchmark's floor kernels (libi4s_floor.so): exported, and argument
    errors are reported before anything is launched (no device needed)."""
    import ctypes
    from int4_sparse_gemv_amd import build as BLD
    out = subprocess.run(["nm", "-D", "--defined-only", BLD.FLOOR_LIB], capture_output=True, text=True).stdout
    names = {l.split()[-1] for l in out.splitlines() if l.strip()}
    assert {"i4sf_stream_read", "i4sf_chase"} <= names
    f = ctypes.CDLL(BLD.FLOOR_LIB)
    f.i4sf_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.i4sf_chase.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    fake = 1 << 20  # never dereferenced: every call below fails its checks first
    assert f.i4sf_stream_read(None, 16, 0, fake, None) == 1
    assert f.i4sf_stream_read(fake, 0, 0, fake, None) == 1
    assert f.i4sf_stream_read(fake, 24, 0, fake, None) == 1      # not a multiple of 16
    assert f.i4sf_stream_read(fake + 4, 16, 0, fake, None) == 1  # misaligned
    assert f.i4sf_chase(None, 16, 10, fake, None) == 1
    assert f.i4sf_chase(fake, 0, 10, fake, None) == 1
    assert f.i4sf_chase(fake, 16, 0, fake, None) == 1
