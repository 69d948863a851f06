"""GPU parity of libi4s against the CPU oracle (needs an MI355X).

Packed buffers must be bit-identical to the oracle's; GEMV outputs must
satisfy |y_gpu - y_ref| <= 1e-3 * sum_j |w_hat_ij x_j| + 1e-5 per element,
where y_ref and the sum come from the oracle in float64.  Every input is
seeded and synthetic (``workloads``).
"""

import sys

import numpy as np
import pytest

import oracle as O
import workloads as WL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module", autouse=True)
def gpu_lib():
    _require_gpu()
    import int4_sparse_gemv_amd as I
    I._binding.load()  # raises if the library is not built
    return I


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_pack(w16, n_keep, g):
    import int4_sparse_gemv_amd as I
    w = torch.from_numpy(w16.view(np.int16)).cuda().view(torch.float16)
    p = I.pack(w, n_keep, g)
    torch.cuda.synchronize()
    return p


def host_bytes(p):
    return {
        "row_ptr": p.row_ptr.cpu().numpy().astype(np.int32),
        "vals": p.vals.cpu().numpy().astype(np.uint8),
        "codes": (p.codes.cpu().numpy().view(np.uint16) if p.codes is not None else np.zeros(0, np.uint16)),
        "scales": p.scales.cpu().numpy().view(np.uint16),
    }


def assert_pack_equal(p, ref, label):
    got = host_bytes(p)
    assert p.group_size == ref["group_size"], f"{label}: G {p.group_size} != {ref['group_size']}"
    for k in ("row_ptr", "vals", "codes", "scales"):
        a, b = got[k], np.asarray(ref[k])
        assert a.shape == b.shape, f"{label}: {k} shape {a.shape} != {b.shape}"
        bad = np.flatnonzero(a != b)
        assert bad.size == 0, f"{label}: {k} differs at {bad.size} positions, first {bad[:5]}"
    if ref["sse"]:
        assert p.sse == ref["sse"], f"{label}: SSE {p.sse} != {ref['sse']}"


def gpu_run(p, x16, use_workspace=True):
    import int4_sparse_gemv_amd as I
    x = torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).cuda().view(torch.float16)
    y = I.run(p, x, use_workspace=use_workspace)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def assert_gemv_close(y_gpu, y_ref, a_ref, label):
    err = np.abs(y_gpu - y_ref)
    tol = 1e-3 * a_ref + 1e-5
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{label}: {len(bad)} outputs outside tolerance, first {bad[:3].tolist()}, "
                           f"max err/tol {float((err / tol).max()):.3g}")


def rand16(rng, shape, scale=0.02):
    return (scale * rng.standard_normal(shape)).astype(np.float16)


# ---------------------------------------------------------------------------
# packer

def test_scale_every_fp16_amax():
    """One row per finite fp16 magnitude: the row's only non-zero is that value."""
    bits = np.arange(0, 0x7C00, dtype=np.uint16)
    w = np.zeros((len(bits), 64), dtype=np.uint16)
    w[:, 5] = bits
    w[1::2, 5] |= 0x8000  # half of them negative
    w16 = w.view(np.float16)
    say(f"case scale-exhaustive rows={len(bits)}")
    ref = O.pack(w16, 4, 64)
    assert_pack_equal(gpu_pack(w16, 4, 64), ref, "scale-exhaustive")


SMALL_CASES = [
    (1, 64, 2, 64), (3, 192, 2, 64), (17, 256, 2, 128), (5, 512, 2, 256), (33, 256, 2, 0),
    (4, 64, 4, 64), (9, 384, 4, 128), (7, 768, 4, 0), (2, 64, 1, 64), (6, 512, 1, 0),
    (11, 1024, 1, 256), (64, 4160, 2, 64),
]


@pytest.mark.parametrize("rows,cols,n_keep,g", SMALL_CASES)
def test_pack_small_with_special_values(rows, cols, n_keep, g):
    rng = np.random.default_rng(rows * 1000 + cols + n_keep)
    w = rand16(rng, (rows, cols))
    # ties, signed zeros, subnormals, extremes and an all-zero row
    w[0, :8] = np.float16([0.5, -0.5, 0.5, -0.5, -0.0, 0.0, 0.0, -0.0])
    if cols >= 32:
        w[0, 8:16] = np.float16([6e-8, -6e-8, 1.2e-7, 0, 65504, -65504, 1, -1])
        w[0, 16:32] = np.float16(rng.integers(-2, 3, 16))
    if rows > 2:
        w[rows // 2] = 0
    say(f"case pack-small {rows}x{cols} n={n_keep} g={g}")
    ref = O.pack(w, n_keep, g)
    assert_pack_equal(gpu_pack(w, n_keep, g), ref, f"{rows}x{cols} n{n_keep} g{g}")


def test_pack_rejects_nonfinite():
    import int4_sparse_gemv_amd as I
    w = np.zeros((4, 256), np.float16)
    w[2, 100] = np.inf
    say("case pack-nonfinite")
    with pytest.raises(I.I4SError) as e:
        gpu_pack(w, 2, 0)
    assert e.value.status == I._binding.I4S_ERR_NONFINITE_WEIGHT
    w[2, 100] = np.nan
    with pytest.raises(I.I4SError):
        gpu_pack(w, 4, 64)


def gpu_pack_ex(w16, n_keep, g, norm, grad):
    import int4_sparse_gemv_amd as I
    w = torch.from_numpy(w16.view(np.int16)).cuda().view(torch.float16)
    n = torch.from_numpy(norm).cuda() if norm is not None else None
    gr = torch.from_numpy(grad.view(np.int16)).cuda().view(torch.float16) if grad is not None else None
    p = I.pack(w, n_keep, g, col_norm=n, grad=gr)
    torch.cuda.synchronize()
    return p


# rows, cols, n_keep, G, which importance inputs, tie-heavy inputs
IMPORTANCE_CASES = [
    (5, 256, 2, 64, "both", False), (33, 512, 2, 0, "both", False), (17, 384, 1, 128, "norm", False),
    (9, 256, 4, 0, "both", False), (40, 1024, 2, 128, "grad", False), (300, 640, 2, 64, "both", True),
    (64, 4160, 1, 64, "both", True), (7, 768, 2, 256, "norm", True), (130, 512, 1, 0, "grad", True),
]


@pytest.mark.parametrize("rows,cols,n_keep,g,which,ties", IMPORTANCE_CASES)
def test_pack_importance_matches_oracle(rows, cols, n_keep, g, which, ties):
    seed = rows * 7919 + cols + n_keep
    if ties:
        rng = np.random.default_rng(seed)
        w = rng.integers(-3, 4, size=(rows, cols)).astype(np.float16)
    else:
        w = WL.make_weight(rows, cols, seed, outliers=True)
    norm, grad = WL.make_importance_inputs(rows, cols, seed + 1, tie_heavy=ties)
    if which == "norm":
        grad = None
    elif which == "grad":
        norm = None
    say(f"case pack-importance {rows}x{cols} n={n_keep} g={g} {which} ties={ties}")
    ref = O.pack(w, n_keep, g, norm, grad)
    p = gpu_pack_ex(w, n_keep, g, norm, grad)
    assert_pack_equal(p, ref, f"importance {rows}x{cols} n{n_keep} g{g} {which}")
    if rows == 40:
        x = WL.make_x(np.random.default_rng(seed + 2), 3, cols)
        y_ref, a_ref = O.gemv(O.reconstruct(ref), x)
        assert_gemv_close(gpu_run(p, x), y_ref, a_ref, "importance-packed gemv")


def test_pack_importance_special_values():
    rng = np.random.default_rng(77)
    rows, cols = 6, 256
    w = rand16(rng, (rows, cols), 1.0)
    w[0, :4] = np.float16([65504, -65504, 1, 0.5])
    w[1, :8] = np.float16([6e-8, -6e-8, 1e-7, 0, -0.0, 2, 3, 1])
    norm = np.exp2(rng.uniform(-20, 20, cols)).astype(np.float32)
    norm[:4] = np.float32([3.0e38, 3.0e38, 3.0e38, 1.0])      # products past fp32's range -> +inf ties
    norm[4:8] = np.float32([1e-40, 2e-40, -0.0, 1e-45])       # fp32 subnormals and -0
    norm[8:12] = 0.0
    grad = rand16(rng, (rows, cols), 1.0)
    grad[1, :8] = np.float16([6e-8, -6e-8, 0, -0.0, 65504, -65504, 1e-5, 0])
    grad[:, 4:8] = 0                                            # keep the subnormal norms visible
    for n_keep in (1, 2):
        for which in ("norm", "both"):
            gr = grad if which == "both" else None
            say(f"case pack-importance-special n={n_keep} {which}")
            ref = O.pack(w, n_keep, 64, norm, gr)
            assert_pack_equal(gpu_pack_ex(w, n_keep, 64, norm, gr), ref, f"special n{n_keep} {which}")


def test_pack_importance_unit_norms_equal_magnitude_pack():
    rng = np.random.default_rng(78)
    w = rand16(rng, (48, 512))
    w[:, ::5] = np.float16(rng.integers(-2, 3, (48, 103)))     # exact magnitude ties
    say("case pack-importance-unit-norms")
    for n_keep, g in ((1, 64), (2, 0), (2, 256)):
        a = host_bytes(gpu_pack(w, n_keep, g))
        b = host_bytes(gpu_pack_ex(w, n_keep, g, np.ones(512, np.float32), None))
        c = host_bytes(gpu_pack_ex(w, n_keep, g, np.ones(512, np.float32), np.zeros(w.shape, np.float16)))
        for k in a:
            assert np.array_equal(a[k], b[k]) and np.array_equal(a[k], c[k]), k


def test_pack_importance_rejects_bad_inputs():
    import int4_sparse_gemv_amd as I
    rows, cols = 4, 256
    w = np.zeros((rows, cols), np.float16)
    ok_n = np.ones(cols, np.float32)
    ok_g = np.zeros((rows, cols), np.float16)
    say("case pack-importance-bad-inputs")
    for v in (-1.0, -1e-45, np.inf, np.nan):
        n = ok_n.copy()
        n[100] = v
        with pytest.raises(I.I4SError) as e:
            gpu_pack_ex(w, 2, 64, n, None)
        assert e.value.status == I._binding.I4S_ERR_INVALID_ARGUMENT, v
    for v in (np.inf, -np.inf, np.nan):
        g = ok_g.copy()
        g[3, 255] = v
        with pytest.raises(I.I4SError) as e:
            gpu_pack_ex(w, 1, 0, ok_n, g)
        assert e.value.status == I._binding.I4S_ERR_INVALID_ARGUMENT, v
    # a non-finite weight is reported first
    w[1, 7] = np.inf
    n = ok_n.copy()
    n[0] = np.nan
    with pytest.raises(I.I4SError) as e:
        gpu_pack_ex(w, 2, 64, n, None)
    assert e.value.status == I._binding.I4S_ERR_NONFINITE_WEIGHT
    # -0 is an allowed norm
    w[1, 7] = 0
    n = ok_n.copy()
    n[5] = -0.0
    gpu_pack_ex(w, 2, 64, n, ok_g)


def config_matrices():
    # every matrix of the single-layer workloads; the 448 matrices of the two
    # 32-layer stacks are checked by test_gpu_stacks.py
    out = []
    for name in ("c1_512", "c2_4096", "c3_mlp7b", "c5_verify13b", "x1_4096_1to4"):
        for m in WL.WORKLOADS[name].matrices:
            out.append((name, m))
    return out


_REF_CACHE = {}


def reference(name, m):
    key = (name, m.name)
    if key not in _REF_CACHE:
        batch = max(WL.WORKLOADS[name].batches)
        w, x = WL.make_weight_and_x(m, batch)
        _REF_CACHE.clear()
        _REF_CACHE[key] = (w, x, O.pack(w, m.n_keep, m.group_size))
    return _REF_CACHE[key]


@pytest.mark.parametrize("name,m", config_matrices(), ids=lambda v: v if isinstance(v, str) else v.name)
def test_config_pack_and_gemv(name, m):
    say(f"case config {name}/{m.name} {m.rows}x{m.cols} n={m.n_keep} g={m.group_size}")
    w, x, ref = reference(name, m)
    p = gpu_pack(w, m.n_keep, m.group_size)
    assert_pack_equal(p, ref, f"{name}/{m.name}")
    w_hat = O.reconstruct(ref)
    for batch in WL.WORKLOADS[name].batches:
        say(f"  gemv batch={batch}")
        y_ref, a_ref = O.gemv(w_hat, x[:batch])
        assert_gemv_close(gpu_run(p, x[:batch]), y_ref, a_ref, f"{name}/{m.name} b{batch}")


# ---------------------------------------------------------------------------
# GEMV edge cases

@pytest.mark.parametrize("rows,cols,n_keep,g", [
    (1, 64, 2, 64), (17, 192, 2, 64), (33, 4160, 2, 64), (100, 8192, 2, 128), (5, 64, 4, 64),
    (19, 320, 4, 64), (21, 4224, 4, 128), (3, 128, 1, 64), (13, 4352, 1, 256), (16, 16384, 2, 256),
    (700, 16384, 1, 128), (9, 20480, 1, 64), (37, 12288, 1, 64), (8200, 1024, 1, 64), (8210, 1024, 2, 128),
    # dense on the matrix cores: two tiles per wave (>= 300 tiles), and two chunks per wave
    (4900, 2048, 4, 64), (40, 13824, 4, 128),
    # K > 16384 on the matrix cores: four chunks per wave
    (24, 20480, 4, 128), (17, 32768, 4, 64), (33, 32768, 1, 256),
    # four tiles per wave at batch > 8 (2:4, >= 640 tiles, K <= 5632), ragged;
    # at K = 4096 it also reads its B fragments compactly; 1:4 of that height
    # takes two tiles of 16-unit chunks there
    (10241, 5632, 2, 256), (10241, 2048, 1, 64), (10241, 4096, 2, 128)])
def test_gemv_shapes_and_all_batches(rows, cols, n_keep, g):
    rng = np.random.default_rng(rows + cols)
    w = rand16(rng, (rows, cols))
    w[rows // 2] = 0  # an all-pruned row
    say(f"case gemv-shape {rows}x{cols} n={n_keep} g={g}")
    ref = O.pack(w, n_keep, g)
    p = gpu_pack(w, n_keep, g)
    assert_pack_equal(p, ref, "shape")
    w_hat = O.reconstruct(ref)
    x = rng.standard_normal((16, cols)).astype(np.float16)
    for batch in range(1, 17):
        y_gpu = gpu_run(p, x[:batch])
        y_ref, a_ref = O.gemv(w_hat, x[:batch])
        assert_gemv_close(y_gpu, y_ref, a_ref, f"b{batch}")
        assert (y_gpu[:, rows // 2] == 0).all()


@pytest.mark.parametrize("R,K,n_keep", [(65535, 32768, 4), (131071, 32768, 2), (65535, 65536, 2),
                                         (32767, 65536, 4), (65535, 65536, 1)])
def test_largest_layer_sampled_rows(R, K, n_keep):
    """The largest layers the format allows, G = 128: dense INT4 with 65535
    rows of 32768 or 32767 of 65536, 2:4 with 131071 rows of 32768 or 65535
    of 65536, so nnz = R * K * N / 4 sits just below 2**31 (as does row_ptr's
    last entry); and 1:4 with 65535 rows of 65536 (2**30 - 16384).  Packed and multiplied on the GPU in full, with and without a
    workspace (K = 65536 splits K across blocks with one).  At a fixed G every
    row packs on its own, so sampled rows (first and last, both sides of tile
    and block edges, random ones) are checked bit for bit against the
    oracle's pack of those rows alone, and their outputs against the oracle's
    GEMV of those rows, at batch 1, 4 and 16 (the last tile of 16 rows is one
    row short)."""
    import int4_sparse_gemv_amd as I
    G = 128
    nnz_row = K * n_keep // 4
    say(f"case largest layer {R}x{K} n={n_keep} G={G}")
    w = WL.make_weight_on_device(R, K, 11, "cuda")
    p = I.pack(w, n_keep, G)
    torch.cuda.synchronize()
    assert p.nnz == R * nnz_row < 2 ** 31
    rng = np.random.default_rng(12)
    half = R // 2
    sel = np.unique(np.concatenate([[0, 1, 15, 16, 255, 256, 8191, 8192, half - 1, half, R - 16, R - 15, R - 1],
                                    rng.integers(0, R, 8)]))
    # every sampled row exists: the gathers below have no bounds check
    assert sel.min() >= 0 and sel.max() < R
    sel_t = torch.from_numpy(sel).cuda()
    w_sel = w[sel_t].cpu().numpy()
    del w
    torch.cuda.empty_cache()
    say("  packed; oracle on the sampled rows")
    ref = O.pack(w_sel, n_keep, G)
    rp = p.row_ptr.cpu().numpy().astype(np.int64)
    np.testing.assert_array_equal(rp, np.arange(R + 1, dtype=np.int64) * nnz_row)
    got = {"vals": p.vals.view(R, nnz_row // 2)[sel_t].cpu().numpy(),
           "scales": p.scales.view(R, K // G)[sel_t].cpu().numpy().view(np.uint16)}
    if n_keep < 4:
        got["codes"] = p.codes.view(R, nnz_row // 8)[sel_t].cpu().numpy().view(np.uint16)
    for k, a in got.items():
        np.testing.assert_array_equal(a, np.asarray(ref[k]).reshape(len(sel), -1), err_msg=k)
    w_hat = O.reconstruct(ref)
    x16 = WL.make_x(np.random.default_rng(13), 16, K)
    for b in (1, 4, 16):
        say(f"  gemv batch={b}")
        y_ref, a_ref = O.gemv(w_hat, x16[:b])
        for ws in ((True, False) if b > 1 else (True,)):
            y = gpu_run(p, x16[:b], use_workspace=ws)
            assert_gemv_close(y[:, sel], y_ref, a_ref, f"largest layer b{b} ws={ws}")


def test_gemv_zero_x_and_unit_vectors():
    rng = np.random.default_rng(77)
    rows, cols = 40, 512
    w = rand16(rng, (rows, cols))
    say("case gemv-unit-vectors")
    ref = O.pack(w, 2, 128)
    p = gpu_pack(w, 2, 128)
    w_hat = O.reconstruct(ref)
    assert (gpu_run(p, np.zeros((3, cols), np.float16)) == 0).all()
    cols_to_try = [0, 1, 2, 3, 63, 64, 255, 256, 511]
    for j0 in range(0, len(cols_to_try), 16):
        js = cols_to_try[j0:j0 + 16]
        x = np.zeros((len(js), cols), np.float16)
        for b, j in enumerate(js):
            x[b, j] = 1.0
        y = gpu_run(p, x)
        for b, j in enumerate(js):
            # a single product s*q is exact in fp32 and rounds once to fp16
            np.testing.assert_array_equal(y[b], w_hat[:, j].astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("rows,cols,n_keep", [(300, 4096, 2), (300, 4096, 1), (300, 4096, 4), (70, 20480, 2),
                                          (40, 40960, 2), (40, 40960, 4)])
def test_all_pruned_rows_give_exact_zero(rows, cols, n_keep):
    """A row that is zero (every group all-pruned: scale +0, q = 0) gives
    y = 0 exactly, and so does a zero quantization group inside a row, on
    every kernel: batch 1 (both forms), batch 2, the matrix-core batch forms,
    the K-split and the VALU batch kernel."""
    rng = np.random.default_rng(rows + cols + n_keep)
    w = rand16(rng, (rows, cols))
    zero_rows = [0, 1, 17, rows // 2, rows - 1]
    w[zero_rows] = 0
    w[5, 128:384] = 0  # whole groups of row 5 (every G divides 128 and 256)
    say(f"case all-pruned rows {rows}x{cols} n={n_keep}")
    p = gpu_pack(w, n_keep, 128)
    ref = O.pack(w, n_keep, 128)
    assert_pack_equal(p, ref, "all-pruned rows")
    w_hat = O.reconstruct(ref)
    assert (w_hat[zero_rows] == 0).all()
    x16 = rng.standard_normal((16, cols)).astype(np.float16)
    for batch in (1, 2, 3, 8, 16):
        y_ref, a_ref = O.gemv(w_hat, x16[:batch])
        for ws in ((True, False) if batch > 1 else (True,)):
            y = gpu_run(p, x16[:batch], use_workspace=ws)
            assert (y[:, zero_rows] == 0).all(), f"b{batch} ws={ws}: nonzero output for an all-pruned row"
            assert_gemv_close(y, y_ref, a_ref, f"all-pruned rows b{batch} ws={ws}")


@pytest.mark.parametrize("n_keep", [1, 2, 4])
def test_batch_rows_match_single_calls(n_keep):
    """Row b of a batch call matches the batch-1 call on x_b (within the
    tolerance: batch 1, batch 2 and batch >= 3 run different kernels here),
    and a row does not depend on the other vectors of its batch: bit-identical
    across every batch size that runs the same kernel shape (batch 3-8 and
    batch 9-16: this layer's one-tile blocks take 8-unit chunks up to 8
    vectors and 16-unit chunks above, which groups the partial sums
    differently; with or without a workspace: at this K the workspace path
    runs the same kernel)."""
    rng = np.random.default_rng(78)
    rows, cols = 64, 2048
    w = rand16(rng, (rows, cols))
    say(f"case gemv-batch-consistency n={n_keep}")
    ref = O.pack(w, n_keep, 64)
    p = gpu_pack(w, n_keep, 64)
    w_hat = O.reconstruct(ref)
    x = rng.standard_normal((16, cols)).astype(np.float16)
    y16 = gpu_run(p, x)
    for b in range(16):
        y1 = gpu_run(p, x[b:b + 1])[0]
        y_ref, a_ref = O.gemv(w_hat, x[b:b + 1])
        assert_gemv_close(y1[None], y_ref, a_ref, f"single {b}")
        assert_gemv_close(y16[b][None], y_ref, a_ref, f"batch row {b}")
    plain16 = gpu_run(p, x, use_workspace=False)
    for b in range(16):
        y_ref, a_ref = O.gemv(w_hat, x[b:b + 1])
        assert_gemv_close(plain16[b][None], y_ref, a_ref, f"no-workspace batch row {b}")
    y2 = gpu_run(p, x[:2], use_workspace=False)
    for b in range(2):
        y_ref, a_ref = O.gemv(w_hat, x[b:b + 1])
        assert_gemv_close(y2[b][None], y_ref, a_ref, f"batch-2 row {b}")
    plain8 = gpu_run(p, x[:8], use_workspace=False)
    for nb in range(3, 8):
        np.testing.assert_array_equal(gpu_run(p, x[:nb], use_workspace=False), plain8[:nb])
    for nb in range(9, 16):
        np.testing.assert_array_equal(gpu_run(p, x[:nb], use_workspace=False), plain16[:nb])
    for nb in range(9, 16):
        np.testing.assert_array_equal(gpu_run(p, x[:nb]), y16[:nb])


# layers of one fused call: (rows, n_keep, G) per layer, K, batch
MULTI_CASES = [
    ([(512, 2, 128), (1000, 2, 128), (777, 2, 128)], 4096, 1),     # q/k/v-like, fused batch-1
    ([(8200, 4, 64), (300, 4, 64)], 1024, 1),                     # dense, two rows per wave
    ([(100, 1, 64), (33, 1, 64), (257, 1, 64)], 2048, 1),         # 1:4, fused batch-1
    ([(512, 2, 128), (1000, 2, 128), (777, 2, 128)], 4096, 5),     # fused matrix-core batch
    ([(200, 1, 256), (70, 1, 256)], 3072, 16),                    # 1:4 fused matrix-core batch
    ([(96, 4, 64), (50, 4, 64)], 1024, 8),                        # dense batch: fused on the matrix cores
    ([(64, 2, 64), (80, 2, 128)], 1024, 1),                       # group sizes differ: per layer
    ([(40, 2, 64)] * 8, 512, 3),                                  # the most layers
    ([(24, 2, 64), (40, 2, 64)], 20480, 1),                       # K > 16384: per layer
    ([(24, 2, 64), (40, 2, 64)], 20480, 4),                       # K > 16384, batch: fused
    ([(512, 2, 128), (1000, 2, 128)], 4096, 2),                   # batch 2: per layer (VALU kernel)
    ([(64, 2, 128), (9000, 2, 128)], 4096, 2),                    # one layer too tall for it: per layer
    ([(24, 2, 64), (40, 2, 64)], 40960, 4),                       # K > 32768: per layer
    ([(4100, 2, 64), (4200, 2, 64)], 1024, 6),                    # two tiles per wave, ragged
    ([(4100, 1, 128), (4200, 1, 128)], 2048, 9),                  # the same for 1:4
    ([(2400, 2, 128), (2400, 2, 128)], 2048, 4),                  # fused at the single calls' chunk width
    ([(10241, 2, 128), (10241, 2, 128)], 2048, 16),               # four tiles per wave, fused
    ([(10241, 1, 64), (10241, 1, 64)], 2048, 12),                 # the same for 1:4
    ([(10241, 2, 128), (600, 2, 128)], 2048, 16),                 # chunk widths differ: per layer
]


@pytest.mark.parametrize("layers,cols,batch", MULTI_CASES)
def test_run_multi_equals_single_calls(layers, cols, batch):
    import int4_sparse_gemv_amd as I
    rng = np.random.default_rng(cols + batch + len(layers))
    say(f"case run-multi {layers} K={cols} b={batch}")
    packs, refs = [], []
    for rows, n_keep, g in layers:
        w = rand16(rng, (rows, cols))
        ref = O.pack(w, n_keep, g)
        p = gpu_pack(w, n_keep, g)
        assert_pack_equal(p, ref, "multi pack")
        packs.append(p)
        refs.append(ref)
    x16 = rng.standard_normal((batch, cols)).astype(np.float16)
    x = torch.from_numpy(x16.view(np.int16)).cuda().view(torch.float16)
    outs = I.run_multi(packs, x)
    singles = [I.run(p, x, use_workspace=False) for p in packs]
    torch.cuda.synchronize()
    for m, (o, s1, ref) in enumerate(zip(outs, singles, refs)):
        got = o.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), s1.cpu().numpy().view(np.uint16)), f"layer {m} differs from i4s_run"
        y_ref, a_ref = O.gemv(O.reconstruct(ref), x16)
        assert_gemv_close(got.astype(np.float64), y_ref, a_ref, f"multi layer {m}")


def test_binding_rejects_bad_outputs_before_any_launch():
    """The Python layer refuses outputs of the wrong shape, dtype or layout
    (the C ABI cannot see a tensor's size) and a workspace on no device."""
    import int4_sparse_gemv_amd as I
    rng = np.random.default_rng(5)
    p = gpu_pack(rand16(rng, (40, 256)), 2, 64)
    x = torch.from_numpy(rng.standard_normal((3, 256)).astype(np.float16)).cuda()
    bad = [torch.empty(3, 39, dtype=torch.float16, device="cuda"),
           torch.empty(3, 40, dtype=torch.float32, device="cuda"),
           torch.empty(40, 3, dtype=torch.float16, device="cuda").t(),
           torch.empty(2, 40, dtype=torch.float16, device="cuda")]
    for o in bad:
        with pytest.raises(ValueError):
            I.run(p, x, out=o)
        with pytest.raises(ValueError):
            I.run_multi([p, p], x, outs=[o, torch.empty(3, 40, dtype=torch.float16, device="cuda")])
    with pytest.raises(ValueError):
        I.run_multi([p, p], x, outs=[torch.empty(3, 40, dtype=torch.float16, device="cuda")])
    with pytest.raises(ValueError):
        I.run(p, x.cpu())
    good = torch.empty(3, 40, dtype=torch.float16, device="cuda")
    I.run(p, x, out=good)
    torch.cuda.synchronize()


def test_run_on_side_stream():
    import int4_sparse_gemv_amd as I
    rng = np.random.default_rng(79)
    rows, cols = 256, 1024
    w = rand16(rng, (rows, cols))
    say("case gemv-side-stream")
    ref = O.pack(w, 2, 128)
    x16 = rng.standard_normal((4, cols)).astype(np.float16)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        wt = torch.from_numpy(w.view(np.int16)).cuda().view(torch.float16)
        p = I.pack(wt, 2, 128)
        x = torch.from_numpy(x16.view(np.int16)).cuda().view(torch.float16)
        y = I.run(p, x)
    s.synchronize()
    y_ref, a_ref = O.gemv(O.reconstruct(ref), x16)
    assert_gemv_close(y.cpu().numpy().astype(np.float64), y_ref, a_ref, "side-stream")


@pytest.mark.parametrize("n_keep,batch,rows,cols", [
    (2, 1, 37, 5120), (4, 1, 37, 5120), (2, 3, 37, 5120), (1, 1, 37, 5120), (4, 8, 37, 5120), (1, 6, 37, 5120),
    # batch 2 on the VALU kernel (each unit decoded once for both vectors)
    (2, 2, 37, 5120), (1, 2, 37, 5120), (4, 2, 37, 5120),
    # more than 8192 rows: two rows per wave at batch 1
    (2, 1, 8200, 1024), (1, 1, 8200, 1024), (4, 1, 8200, 2048),
    # layers whose workspace path splits K (batch 3-8 with long rows on few
    # rows, batch 16, K > 32768): the split kernel's per-lane recompute
    (2, 8, 300, 8192), (2, 16, 37, 13824), (2, 4, 40, 40960)])
def test_row_ptr_is_honoured(n_keep, batch, rows, cols):
    """Rows stored in reverse order, described only by row_ptr, give the same y
    (bit for bit on the VALU kernels, within the tolerance on the matrix cores)."""
    import int4_sparse_gemv_amd as I
    rng = np.random.default_rng(80 + n_keep)
    g = 128
    w = rand16(rng, (rows, cols))
    say(f"case row-ptr-reversed n={n_keep} b={batch} {rows}x{cols}")
    p = gpu_pack(w, n_keep, g)
    x16 = rng.standard_normal((batch, cols)).astype(np.float16)
    y0 = gpu_run(p, x16)
    nnz_row = cols * n_keep // 4
    vb, cb = nnz_row // 2, nnz_row // 8
    perm = torch.arange(rows - 1, -1, -1, device=p.vals.device)
    vals = p.vals.view(rows, vb)[perm].reshape(-1).contiguous()
    codes = p.codes.view(rows, cb)[perm].reshape(-1).contiguous() if p.codes is not None else None
    row_ptr = torch.tensor([(rows - 1 - i) * nnz_row for i in range(rows)] + [rows * nnz_row],
                           dtype=torch.int32, device=p.vals.device)
    q = I.PackedWeight(rows, cols, n_keep, p.group_size, row_ptr, vals, codes, p.scales)
    y1 = gpu_run(q, x16)
    if batch <= 2:
        # the VALU kernels recompute a moved row with the same arithmetic
        np.testing.assert_array_equal(y0, y1)
    else:
        # the matrix-core kernel recomputes it with a per-lane loop: within
        # the tolerance, not necessarily the same bits
        ref = O.pack(w, n_keep, g)
        y_ref, a_ref = O.gemv(O.reconstruct(ref), x16)
        assert_gemv_close(y1, y_ref, a_ref, f"row-ptr-reversed n={n_keep} b={batch}")


@pytest.mark.parametrize("rows,cols,batch,g", [
    (200, 2048, 3, 64), (5120, 1024, 16, 64), (128, 13824, 16, 64), (777, 4352, 8, 64), (8200, 1024, 4, 64),
    (300, 8192, 8, 64), (8193, 2048, 16, 64), (64, 5120, 4, 128), (48, 2048, 2, 128), (40, 16384, 8, 128),
    (64, 5120, 4, 256), (33, 13824, 16, 256), (16, 1024, 5, 128),
    # two-tile blocks fewer than the compute units at batch <= 8: 8-unit chunks
    (6000, 2048, 6, 128), (5000, 3072, 3, 64),
    # K > 16384: four chunks per wave at batch <= 8; the workspace path splits
    # K across blocks at batch > 8 on few rows and for any batch beyond 32768
    (96, 20480, 5, 64), (300, 24576, 16, 128), (40, 32768, 9, 256), (64, 40960, 4, 128),
    # K split with two tiles per wave, a partial last tile and a partial last
    # row group (and at 13824 columns a half-width last slice); 4500 rows: 36
    # row groups, so the sum's blocks past the last multiple of 8 groups take
    # the remaining 4 groups (two blocks each)
    (5000, 13824, 8, 256), (8100, 7168, 16, 64), (4500, 13824, 16, 128)])
def test_batch_paths_with_and_without_workspace(rows, cols, batch, g):
    """i4s_run (no workspace) and i4s_run_ws (K split across blocks where the
    layer's plan uses it) both meet the tolerance for every group size; the
    workspace path is deterministic across repeated calls."""
    import int4_sparse_gemv_amd as I
    rng = np.random.default_rng(rows + batch + g)
    w = rand16(rng, (rows, cols))
    say(f"case batch-paths {rows}x{cols} b{batch} G{g}")
    ref = O.pack(w, 2, g)
    p = gpu_pack(w, 2, g)
    w_hat = O.reconstruct(ref)
    x16 = rng.standard_normal((batch, cols)).astype(np.float16)
    y_ref, a_ref = O.gemv(w_hat, x16)
    x = torch.from_numpy(x16.view(np.int16)).cuda().view(torch.float16)
    y_plain = I.run(p, x, use_workspace=False)
    y_ws1 = I.run(p, x)
    y_ws2 = I.run(p, x)
    torch.cuda.synchronize()
    for y in (y_plain, y_ws1):
        assert_gemv_close(y.cpu().numpy().astype(np.float64), y_ref, a_ref, f"{rows}x{cols} b{batch}")
    assert torch.equal(y_ws1, y_ws2)


def test_shared_workspace_across_layers_and_graph_replay():
    """One workspace serves different layers in turn, whatever it holds on
    entry, also when the calls are replayed from a graph."""
    import int4_sparse_gemv_amd as I
    rng = np.random.default_rng(91)
    shapes = [(640, 20480), (1536, 1024), (96, 24576), (8320, 512)]  # two of them split K
    packs, xs, refs = [], [], []
    for r, c in shapes:
        w = rand16(rng, (r, c))
        ref = O.pack(w, 2, 128)
        packs.append(gpu_pack(w, 2, 128))
        x16 = rng.standard_normal((16, c)).astype(np.float16)
        xs.append(torch.from_numpy(x16.view(np.int16)).cuda().view(torch.float16))
        refs.append(O.gemv(O.reconstruct(ref), x16))
    say("case shared-workspace")
    need = max(I.run_workspace_size(p, 16) for p in packs)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bytes: must not matter
    outs = [torch.empty(16, r, dtype=torch.float16, device="cuda") for r, _ in shapes]
    for _ in range(2):
        for p, x, o in zip(packs, xs, outs):
            I.run(p, x, out=o, workspace=ws)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for o, (y_ref, a_ref) in zip(eager, refs):
        assert_gemv_close(o.cpu().numpy().astype(np.float64), y_ref, a_ref, "shared workspace")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        descs = [p.descriptor() for p in packs]
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for p, x, o, d in zip(packs, xs, outs, descs):
                I.run(p, x, out=o, descriptor=d, workspace=ws)
    for _ in range(3):
        for o in outs:
            o.zero_()
        ws.fill_(0xFF)
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e)


def _decode_layer(I, packs, xs, outs):
    """One decoder layer's calls: q/k/v fused, o, gate/up fused, down."""
    q, k, v, o, g, u, d = packs
    I.run_multi([q, k, v], xs[0], outs=outs[0:3])
    I.run(o, xs[1], out=outs[3], use_workspace=False)
    I.run_multi([g, u], xs[2], outs=outs[4:6])
    I.run(d, xs[3], out=outs[6], use_workspace=False)


@pytest.mark.parametrize("batch", [1, 4])
def test_decode_layer_graph_replay(batch):
    """A layer's sequence of calls captured in a HIP graph replays to the
    eager result, bit for bit, with eager work between the replays."""
    import int4_sparse_gemv_amd as I
    rng = np.random.default_rng(300 + batch)
    shapes = [(512, 1024, 2)] * 4 + [(1536, 1024, 2), (1536, 1024, 2), (1024, 1536, 1)]  # q k v o gate up down
    packs, refs = [], []
    for r, c, nk in shapes:
        w = rand16(rng, (r, c))
        ref = O.pack(w, nk, 64)
        packs.append(gpu_pack(w, nk, 64))
        refs.append(ref)
    x16 = [rng.standard_normal((batch, c)).astype(np.float16) for c in (1024, 1024, 1024, 1536)]
    xs = [torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16) for a in x16]
    outs = [torch.empty(batch, r, dtype=torch.float16, device="cuda") for r, _, _ in shapes]
    say(f"case decode-layer-graph b{batch}")
    _decode_layer(I, packs, xs, outs)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    xin = [x16[0]] * 3 + [x16[1]] + [x16[2]] * 2 + [x16[3]]
    for m, (e, ref) in enumerate(zip(eager, refs)):
        y_ref, a_ref = O.gemv(O.reconstruct(ref), xin[m])
        assert_gemv_close(e.cpu().numpy().astype(np.float64), y_ref, a_ref, f"layer call {m}")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            _decode_layer(I, packs, xs, outs)
    for _ in range(3):
        for o in outs:
            o.fill_(7)
        _decode_layer(I, packs, xs, [torch.empty_like(o) for o in outs])  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e)


_FIRST_LAUNCH_IN_CAPTURE = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
import int4_sparse_gemv_amd as I
rng = np.random.default_rng(5)
# 5120 x 5120 at batch 4: the two-tile, 8-unit batch kernel with 10 waves,
# whose 74 KB of LDS needs the per-kernel limit raised; its first launch is
# the captured one
w = torch.from_numpy((0.02 * rng.standard_normal((5120, 5120))).astype(np.float16).view(np.int16)).cuda().view(torch.float16)
p = I.pack(w, 2, 64)
x = torch.from_numpy(rng.standard_normal((4, 5120)).astype(np.float16).view(np.int16)).cuda().view(torch.float16)
out = torch.empty(4, 5120, dtype=torch.float16, device="cuda")
d = p.descriptor()
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
side = torch.cuda.Stream()
with torch.cuda.stream(side):
    with torch.cuda.graph(g, stream=side):
        I.run(p, x, out=out, descriptor=d, use_workspace=False)
out.zero_()
g.replay()
torch.cuda.synchronize()
ref = I.run(p, x, use_workspace=False)
torch.cuda.synchronize()
assert torch.equal(out, ref), "captured first launch differs from the eager call"
print("ok", flush=True)
"""


def test_first_launch_of_a_kernel_inside_graph_capture():
    """The first launch of a batch kernel that needs more than 64 KB of LDS
    may happen inside a graph capture (a fresh process makes it the first)."""
    import os
    import subprocess
    say("case first-launch-in-capture (subprocess)")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_LAUNCH_IN_CAPTURE, root], capture_output=True, text=True,
                       timeout=110)
    assert r.returncode == 0 and "ok" in r.stdout, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
