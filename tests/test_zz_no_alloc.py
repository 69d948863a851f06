"""i4s_run_noalloc, the entry point that allocates nothing, against i4s_run_ws.

Called through the C ABI (ctypes).  Both run the same kernels; the
no-allocation form takes its K-split partial sums from the library's static
per-GPU scratch array instead of a caller workspace, so the outputs must be
identical bit for bit.  Two calls in a row, the second on a smaller layer
and batch, so the second reads the array after the first has left its
partial sums there.  Every case here splits K (the workspace size is
nonzero), and the layer whose workspace exceeds the array is refused before
anything is enqueued.
"""

import ctypes
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_sparse_gemv_amd as I
    return I._binding.load()


def packed_layer(rows, cols, n_keep, g, seed):
    import int4_sparse_gemv_amd as I
    rng = np.random.default_rng(seed)
    w16 = (0.02 * rng.standard_normal((rows, cols))).astype(np.float16)
    w = torch.from_numpy(w16.view(np.int16)).cuda().view(torch.float16)
    p = I.pack(w, n_keep, g)
    x16 = rng.standard_normal((16, cols)).astype(np.float16)
    x = torch.from_numpy(x16.view(np.int16)).cuda().view(torch.float16)
    return p, x


def both(lib, p, x, batch):
    """(y from i4s_run_noalloc, y from i4s_run_ws, workspace bytes)."""
    from int4_sparse_gemv_amd import _binding as B
    d = p.descriptor()
    need = ctypes.c_uint64()
    B.check(lib.i4s_run_workspace_size(ctypes.byref(d), batch, ctypes.byref(need)), "i4s_run_workspace_size")
    sh = torch.cuda.current_stream().cuda_stream
    xb = x[:batch].contiguous()
    y_na = torch.full((batch, p.rows), float("nan"), dtype=torch.float16, device="cuda")
    y_ws = torch.full((batch, p.rows), float("nan"), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device="cuda")
    B.check(lib.i4s_run_noalloc(ctypes.byref(d), xb.data_ptr(), batch, y_na.data_ptr(), sh), "i4s_run_noalloc")
    B.check(lib.i4s_run_ws(ctypes.byref(d), xb.data_ptr(), batch, y_ws.data_ptr(), ws.data_ptr(), ws.numel(), sh),
            "i4s_run_ws")
    torch.cuda.synchronize()
    return y_na.cpu().numpy().view(np.uint16), y_ws.cpu().numpy().view(np.uint16), need.value


def test_noalloc_equals_workspace_call_twice_second_smaller(lib):
    # 2:4 with K > 32768 splits K across blocks at every batch >= 2
    first = (4096, 40960, 2, 128, 8)      # rows, cols, n_keep, G, batch
    second = (1000, 36864, 2, 64, 3)
    for rows, cols, n_keep, g, batch in (first, second):
        say(f"case noalloc {rows}x{cols} n={n_keep} G={g} b={batch}")
        p, x = packed_layer(rows, cols, n_keep, g, rows + cols)
        y_na, y_ws, need = both(lib, p, x, batch)
        assert need > 0, "the case must use the scratch (a K split)"
        assert not np.isnan(y_na.view(np.float16)).any()
        np.testing.assert_array_equal(y_na, y_ws)


def test_noalloc_without_split_and_batch_one(lib):
    """Calls that need no workspace run the same kernels as i4s_run."""
    for rows, cols, n_keep, g, batch in ((512, 4096, 2, 128, 1), (300, 2048, 1, 64, 5), (64, 1024, 4, 64, 16)):
        say(f"case noalloc no-split {rows}x{cols} n={n_keep} b={batch}")
        p, x = packed_layer(rows, cols, n_keep, g, rows * 3 + cols)
        y_na, y_ws, need = both(lib, p, x, batch)
        assert need == 0
        np.testing.assert_array_equal(y_na, y_ws)


def test_noalloc_refuses_a_workspace_beyond_the_array(lib):
    """A layer whose K split needs more than the static array is refused on
    the host, before any launch (descriptor only: no buffers are read)."""
    from int4_sparse_gemv_amd import _binding as B
    say("case noalloc too large")
    rows, cols, batch = 16384, 65536, 16
    d = B.i4s_packed()
    d.rows, d.cols, d.n_keep, d.group_size = rows, cols, 2, 128
    d.nnz = rows * cols // 2
    need = ctypes.c_uint64()
    B.check(lib.i4s_run_workspace_size(ctypes.byref(d), batch, ctypes.byref(need)), "i4s_run_workspace_size")
    assert need.value > B.I4S_NOALLOC_SCRATCH_BYTES
    # buffers of the descriptor's sizes (never read: the call is refused first)
    sz = B.i4s_sizes()
    B.check(lib.i4s_pack_sizes(rows, cols, 2, 128, ctypes.byref(sz)), "i4s_pack_sizes")
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda") for n in (sz.row_ptr, sz.vals, sz.codes, sz.scales)]
    d.row_ptr, d.vals, d.codes, d.scales = [b.data_ptr() for b in bufs]
    x = torch.empty(batch, cols, dtype=torch.float16, device="cuda")
    y = torch.empty(batch, rows, dtype=torch.float16, device="cuda")
    st = lib.i4s_run_noalloc(ctypes.byref(d), x.data_ptr(), batch, y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == B.I4S_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
