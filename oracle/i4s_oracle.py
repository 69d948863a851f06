"""CPU oracle for the INT4 2-bit-CSR SparseGEMV.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module: only the test suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP library (no kernels, headers,
tables or helpers) and it never reads anything the GPU produced as an input.

Source of every rule below: "Efficient LLM-based Advertising via Model
Compression and Parallel Verification" (arXiv 2605.11582).
  * Section 3.2, "Sparsification" and Eq. (3): the element importance is
    |W_ij|*||X_j||_2 + |W_ij|*|dE/dW_ij|; the N:4 mask keeps, per aligned group
    of four columns, the N most important elements.  Without supplied
    activation norms and gradients (a constant norm, no gradient term) it
    orders elements by |W_ij| (magnitude pruning); with them, by the score
    below.
  * Section 3.2, "Adaptive Group-Wise Quantization" and section 3.1: INT4
    weight-only quantization in groups whose size is chosen per layer.  The
    page does not give the selection rule; this oracle picks, per matrix, the
    group size in {64, 128, 256} with the smallest exact reconstruction
    squared error, ties going to the larger group.
  * Section 3.3, "Sparse Index Structure" and "Computational Acceleration",
    and the first contribution bullet of section 1: the kept elements are
    stored CSR-style, each with a 2-bit in-group column index; the indices
    are packed into uint16 words starting from the least significant bits;
    the index plus weight bytes come to 30 % of a plain CSR.
  * Section 3.3: the weights are INT4 and are widened to fp16 inside the
    kernel; this oracle reconstructs them exactly in float64 instead.

Readings taken where the page is silent (each is also listed with the design
notes of the repository):
  * G counts dense columns along K; a quant group holds G*N/4 stored elements.
  * symmetric INT4: s = fp16_RNE(amax / 7); q = clamp(round_half_even(w / s),
    -8, 7); q = 0 where s == 0; the stored nibble is q + 8.
  * pruning happens on the fp16 weights before quantization; among equal
    magnitudes (or scores) the lower in-group column is kept; kept columns are
    listed in ascending order.
  * Eq. (3) is evaluated as |W_ij| * (n_j + |g_ij|), factored, in float32: the
    sum n_j + |g_ij| is rounded once to float32 and the product once more
    (round to nearest even).  n_j is the caller's float32 column norm
    ||X_j||_2 (1 when none is given), g_ij the fp16 gradient (0 when none is
    given); norms must be finite and non-negative, gradients finite.  A
    product beyond float32's range is +inf (and ties other +inf scores).  A
    defined precision is needed because the kept set is an exact decision;
    with norms of 1 and no gradients the score is |W_ij| itself.
  * element order inside each 32-bit word of ``vals``: nibble slots 0..7 hold
    elements 0,2,4,6,1,3,5,7 of the word's 8 elements.
  * ``row_ptr[i] = i * K * N / 4`` (every row of an N:4 matrix has the same
    length; an all-zero row is still stored).
  * y = W_hat x is accumulated exactly here (float64); the library rounds it to
    fp16.

Parity of the byte layout with the page is pinned only as far as the page
goes (2 bits per index, 8 indices per uint16, least significant bits first);
the nibble interleave and the exact word layout are this design's own and are
pinned by a hand-derived worked example in the tests.
"""

from __future__ import annotations

from typing import Dict, Iterable, Tuple

import numpy as np

CANDIDATE_GROUP_SIZES = (64, 128, 256)

# element index (0..7) held by nibble slot 0..7 of a 32-bit vals word
SLOT_TO_ELEMENT = (0, 2, 4, 6, 1, 3, 5, 7)


class OracleError(ValueError):
    pass


# --------------------------------------------------------------------------
# validation


def check_args(w16: np.ndarray, n_keep: int, group_size: int, col_norm=None, grad16=None) -> None:
    if w16.dtype != np.float16 or w16.ndim != 2:
        raise OracleError("W must be a 2-D float16 array")
    rows, cols = w16.shape
    if rows < 1 or cols < 64 or cols % 64:
        raise OracleError("need rows >= 1 and cols a positive multiple of 64")
    if n_keep not in (1, 2, 4):
        raise OracleError("n_keep must be 1, 2 or 4")
    sizes = CANDIDATE_GROUP_SIZES if group_size == 0 else (group_size,)
    for g in sizes:
        if g not in CANDIDATE_GROUP_SIZES:
            raise OracleError("group size must be 64, 128, 256 or 0 (adaptive)")
        if cols % g:
            raise OracleError(f"cols={cols} is not a multiple of group size {g}")
    if not np.isfinite(w16).all():
        raise OracleError("W has a non-finite entry")
    if col_norm is not None:
        if col_norm.dtype != np.float32 or col_norm.shape != (cols,):
            raise OracleError("column norms must be float32 of shape [cols]")
        if not np.isfinite(col_norm).all() or (col_norm < 0).any():
            raise OracleError("column norms must be finite and non-negative")
    if grad16 is not None:
        if grad16.dtype != np.float16 or grad16.shape != w16.shape:
            raise OracleError("gradients must be float16 of W's shape")
        if not np.isfinite(grad16).all():
            raise OracleError("gradients must be finite")


# --------------------------------------------------------------------------
# step 1: N:4 mask by the importance of Eq. (3)


def importance(w16: np.ndarray, col_norm=None, grad16=None) -> np.ndarray:
    """Eq. (3), |W_ij| * ||X_j||_2 + |W_ij| * |dE/dW_ij|, as float32 scores.

    Evaluated as |W_ij| * (n_j + |g_ij|) with one float32 rounding for the
    sum and one for the product; n_j = 1 without norms, g_ij = 0 without
    gradients.
    """
    rows, cols = w16.shape
    n = np.ones(cols, np.float32) if col_norm is None else col_norm.astype(np.float32)
    g = np.zeros((rows, cols), np.float32) if grad16 is None else np.abs(grad16.astype(np.float32))
    a = (n[None, :] + g).astype(np.float32)  # float32 + float32: one rounding
    with np.errstate(over="ignore"):          # a product past float32's range is +inf
        return (np.abs(w16.astype(np.float32)) * a).astype(np.float32)


def nm_mask(w16: np.ndarray, n_keep: int, col_norm=None, grad16=None) -> np.ndarray:
    """In-group columns kept per aligned group of 4 columns.

    Returns an int array [rows][cols/4][n_keep], ascending along the last
    axis.  The kept set is the n_keep most important elements of the group
    (by |w| when neither norms nor gradients are given, else by the float32
    score of ``importance``); among equal values the smaller in-group column
    wins.
    """
    rows, cols = w16.shape
    if col_norm is None and grad16 is None:
        mag = np.abs(w16.astype(np.float64)).reshape(rows, cols // 4, 4)
    else:
        mag = importance(w16, col_norm, grad16).astype(np.float64).reshape(rows, cols // 4, 4)
    # a stable sort of -|w| lists equal magnitudes in ascending column order
    order = np.argsort(-mag, axis=-1, kind="stable")
    return np.sort(order[..., :n_keep], axis=-1)


def element_stream(w16: np.ndarray, kept: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Kept values (float64) and their dense columns, [rows][nnz_row] each.

    Element e of a row belongs to 4-column group e // N and sits in column
    4 * (e // N) + code_e.
    """
    rows, cols = w16.shape
    n_keep = kept.shape[-1]
    base = (4 * np.arange(cols // 4))[None, :, None]
    col = (base + kept).reshape(rows, -1)
    val = np.take_along_axis(w16.astype(np.float64), col, axis=1)
    return val, col


# --------------------------------------------------------------------------
# steps 2-3: group scale and INT4 quantization


def group_scales(val: np.ndarray, n_keep: int, group_size: int) -> np.ndarray:
    """s = fp16_RNE(amax / 7) per quant group of ``group_size`` dense columns.

    Returns float16 [rows][cols/group_size].  The division is carried out in
    float64 (correctly rounded) and the float64 -> float16 cast rounds to
    nearest even; amax / 7 never lands within float64 rounding distance of an
    fp16 rounding boundary unless it is exact, so the two roundings give the
    single correctly rounded result (the tests check this for every fp16
    amax).
    """
    rows, nnz_row = val.shape
    per_group = group_size * n_keep // 4
    amax = np.abs(val).reshape(rows, nnz_row // per_group, per_group).max(axis=-1)
    return (amax / 7.0).astype(np.float16)


def quantize(val: np.ndarray, scales16: np.ndarray, n_keep: int, group_size: int) -> np.ndarray:
    """q = clamp(round_half_even(w / s), -8, 7), and q = 0 where s == 0."""
    per_group = group_size * n_keep // 4
    s = np.repeat(scales16.astype(np.float64), per_group, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(val / s), -8, 7)
    q = np.where(s == 0.0, 0.0, q)
    return q.astype(np.int64)


# --------------------------------------------------------------------------
# step 4: exact reconstruction error and the per-matrix group size


def _sum_of_squares(n: np.ndarray) -> int:
    """Exact sum of n**2 over an int64 array with |n| < 2**44, as a Python int.

    n = hi * 2**22 + lo with 0 <= lo < 2**22, so
    n**2 = hi**2 * 2**44 + hi*lo * 2**23 + lo**2; each partial product is
    below 2**44 and a row of fewer than 2**19 terms sums inside int64.
    """
    n = np.asarray(n, dtype=np.int64)
    if n.ndim == 1:
        n = n[None, :]
    if n.size == 0:
        return 0
    if int(np.abs(n).max()) >= (1 << 44):
        raise OracleError("error term outside the exact range")
    if n.shape[1] >= (1 << 19):
        raise OracleError("row too long for the exact partial sums")
    lo = n & ((1 << 22) - 1)
    hi = n >> 22
    a = (hi * hi).sum(axis=1).tolist()
    b = (hi * lo).sum(axis=1).tolist()
    c = (lo * lo).sum(axis=1).tolist()
    return sum((ai << 44) + (bi << 23) + ci for ai, bi, ci in zip(a, b, c))


def sse_units(val: np.ndarray, scales16: np.ndarray, q: np.ndarray,
              n_keep: int, group_size: int) -> int:
    """sum_e (w_e - s*q_e)**2 over the kept elements, in units of 2**-48.

    Every fp16 value, and every fp16 scale times a small integer, is an
    integer multiple of 2**-24, so the error terms are exact integers in
    units of 2**-24 and their squares in units of 2**-48.
    """
    per_group = group_size * n_keep // 4
    s = np.repeat(scales16.astype(np.float64), per_group, axis=1)
    w_units = val * 2.0 ** 24                  # exact: |w| <= 65504
    sq_units = s * 2.0 ** 24 * q               # exact: < 2**43
    n = (w_units - sq_units).astype(np.int64)  # exact integer difference
    return _sum_of_squares(n)


def choose_group_size(val: np.ndarray, n_keep: int,
                      candidates: Iterable[int] = CANDIDATE_GROUP_SIZES) -> Tuple[int, Dict[int, int]]:
    """Group size with the smallest exact SSE; ties go to the larger size."""
    sse: Dict[int, int] = {}
    for g in candidates:
        s = group_scales(val, n_keep, g)
        q = quantize(val, s, n_keep, g)
        sse[g] = sse_units(val, s, q, n_keep, g)
    best = None
    for g in sorted(sse, reverse=True):
        if best is None or sse[g] < sse[best]:
            best = g
    return best, sse


# --------------------------------------------------------------------------
# step 5: encode the 2-bit CSR buffers


def encode_vals(q: np.ndarray) -> np.ndarray:
    """Nibbles u = q + 8, eight per little-endian 32-bit word, slot order 0,2,4,6,1,3,5,7."""
    rows, nnz_row = q.shape
    u = (q + 8).astype(np.uint32).reshape(rows, nnz_row // 8, 8)
    word = np.zeros((rows, nnz_row // 8), dtype=np.uint32)
    for slot, elem in enumerate(SLOT_TO_ELEMENT):
        word |= u[..., elem] << np.uint32(4 * slot)
    return word.astype("<u4").view(np.uint8).reshape(-1)


def encode_codes(kept: np.ndarray) -> np.ndarray:
    """2-bit in-group columns, eight per uint16, element e at bits 2*(e % 8)."""
    rows = kept.shape[0]
    c = kept.reshape(rows, -1).astype(np.uint32)
    c = c.reshape(rows, -1, 8)
    word = np.zeros(c.shape[:2], dtype=np.uint32)
    for k in range(8):
        word |= c[..., k] << np.uint32(2 * k)
    return word.astype(np.uint16).reshape(-1)


def pack(w16: np.ndarray, n_keep: int, group_size: int, col_norm=None, grad16=None) -> Dict[str, object]:
    """Prune, quantize and encode W; ``group_size`` 0 picks it per matrix.

    ``col_norm`` (float32 [cols], the activation norms ||X_j||_2) and
    ``grad16`` (float16, W's shape, dE/dW) are the optional inputs of Eq. (3);
    without them the mask is by magnitude.

    Returns a dict with the four buffers (``row_ptr`` int32, ``vals`` uint8,
    ``codes`` uint16 (empty when n_keep == 4), ``scales`` uint16 fp16 bits),
    the shape and pattern, the group size used and, when chosen adaptively,
    the exact SSE of each candidate in units of 2**-48.
    """
    check_args(w16, n_keep, group_size, col_norm, grad16)
    rows, cols = w16.shape
    kept = nm_mask(w16, n_keep, col_norm, grad16)
    val, _ = element_stream(w16, kept)
    sse: Dict[int, int] = {}
    if group_size == 0:
        group_size, sse = choose_group_size(val, n_keep)
    s = group_scales(val, n_keep, group_size)
    q = quantize(val, s, n_keep, group_size)
    nnz_row = cols * n_keep // 4
    return {
        "rows": rows, "cols": cols, "n_keep": n_keep, "group_size": group_size,
        "nnz": rows * nnz_row,
        "row_ptr": (np.arange(rows + 1, dtype=np.int64) * nnz_row).astype(np.int32),
        "vals": encode_vals(q),
        "codes": encode_codes(kept) if n_keep < 4 else np.zeros(0, np.uint16),
        "scales": s.view(np.uint16).reshape(-1).copy(),
        "sse": sse,
    }


# --------------------------------------------------------------------------
# decode and reconstruct (reads only the buffers)


def decode(packed: Dict[str, object]) -> Tuple[np.ndarray, np.ndarray]:
    """(q, code) per stored element, each [rows][nnz_row], from the raw buffers."""
    rows, cols, n_keep = packed["rows"], packed["cols"], packed["n_keep"]
    nnz_row = cols * n_keep // 4
    row_ptr = np.asarray(packed["row_ptr"], dtype=np.int64)
    if row_ptr.shape != (rows + 1,) or row_ptr[0] != 0 or np.any(np.diff(row_ptr) != nnz_row):
        raise OracleError("row_ptr does not describe rows of K*N/4 elements")
    words = np.asarray(packed["vals"], dtype=np.uint8).view("<u4").astype(np.uint32)
    words = words.reshape(rows, nnz_row // 8)
    u = np.zeros((rows, nnz_row // 8, 8), dtype=np.int64)
    for slot, elem in enumerate(SLOT_TO_ELEMENT):
        u[..., elem] = (words >> np.uint32(4 * slot)) & np.uint32(0xF)
    q = (u - 8).reshape(rows, nnz_row)
    if n_keep == 4:
        code = np.broadcast_to(np.arange(nnz_row) % 4, (rows, nnz_row)).astype(np.int64)
    else:
        cw = np.asarray(packed["codes"], dtype=np.uint16).astype(np.uint32).reshape(rows, nnz_row // 8)
        code = np.zeros((rows, nnz_row // 8, 8), dtype=np.int64)
        for k in range(8):
            code[..., k] = (cw >> np.uint32(2 * k)) & np.uint32(3)
        code = code.reshape(rows, nnz_row)
        g = code.reshape(rows, cols // 4, n_keep)
        if n_keep > 1 and np.any(np.diff(g, axis=-1) <= 0):
            raise OracleError("in-group columns are not strictly ascending")
    return q, code


def reconstruct(packed: Dict[str, object]) -> np.ndarray:
    """Dense float64 W_hat [rows][cols]: s_g * q at each stored position, 0 elsewhere."""
    rows, cols, n_keep, gsz = packed["rows"], packed["cols"], packed["n_keep"], packed["group_size"]
    q, code = decode(packed)
    nnz_row = cols * n_keep // 4
    col = 4 * (np.arange(nnz_row) // n_keep)[None, :] + code
    s = np.asarray(packed["scales"], dtype=np.uint16).view(np.float16).astype(np.float64)
    s = s.reshape(rows, cols // gsz)
    s_e = np.take_along_axis(s, col // gsz, axis=1)
    w_hat = np.zeros((rows, cols), dtype=np.float64)
    np.put_along_axis(w_hat, col, s_e * q, axis=1)
    return w_hat


# --------------------------------------------------------------------------
# the GEMV and its tolerance scale


def gemv(w_hat: np.ndarray, x16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """y[b, i] = sum_j W_hat[i, j] * x[b, j] and a[b, i] = sum_j |W_hat[i, j] * x[b, j]|, float64."""
    x = np.atleast_2d(np.asarray(x16)).astype(np.float64)
    return x @ w_hat.T, np.abs(x) @ np.abs(w_hat).T


def run(packed: Dict[str, object], x16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """The oracle's whole call: reconstruct W_hat from the buffers, then the GEMV."""
    return gemv(reconstruct(packed), x16)


# --------------------------------------------------------------------------
# sizes


def packed_nbytes(rows: int, cols: int, n_keep: int, group_size: int) -> Dict[str, int]:
    nnz = rows * cols * n_keep // 4
    return {
        "row_ptr": 4 * (rows + 1),
        "vals": nnz // 2,
        "codes": (nnz // 4) if n_keep < 4 else 0,
        "scales": 2 * rows * (cols // group_size),
    }


def plain_csr_nbytes(nnz: int) -> Dict[str, int]:
    """The uncompressed comparator: INT4 values plus one uint16 column index per element."""
    return {"vals": nnz // 2, "col_idx": 2 * nnz}
