"""INT4 2-bit-CSR SparseGEMV for AMD Instinct MI355X (gfx950).

``pack`` prunes (N:4 by magnitude, or by the full Eq. (3) importance when
column norms and/or gradients are given), quantizes (symmetric INT4, fp16 group
scales, group size fixed or chosen per matrix by minimum SSE) and encodes a
dense fp16 weight; ``run`` computes y = W_hat x for 1-16 fp16 vectors.  Both
call the HIP kernels of ``libi4s.so`` through its C ABI (``include/i4s.h``);
PyTorch only provides device memory and the current stream.  The method is
the one of "Efficient LLM-based Advertising via Model Compression and
Parallel Verification", sections 3.2 and 3.3.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import ctypes

from . import _binding as B
from ._binding import (  # noqa: F401  (the C names)
    I4SError, i4s_format_version, i4s_last_error, i4s_pack, i4s_pack_ex, i4s_pack_sizes, i4s_run,
    i4s_run_multi, i4s_run_workspace_size, i4s_run_ws, i4s_status_string, i4s_version,
)

__all__ = ["PackedWeight", "pack", "run", "run_multi", "pack_sizes", "run_workspace_size", "I4SError",
           "i4s_pack_sizes", "i4s_pack", "i4s_pack_ex", "i4s_run", "i4s_run_multi", "i4s_run_workspace_size", "i4s_run_ws",
           "i4s_status_string", "i4s_last_error", "i4s_version", "i4s_format_version"]


def _torch():
    import torch
    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def pack_sizes(rows: int, cols: int, n_keep: int, group_size: int) -> Dict[str, int]:
    sz = B.i4s_sizes()
    B.check(B.i4s_pack_sizes(rows, cols, n_keep, group_size, sz), "i4s_pack_sizes")
    return {"row_ptr": sz.row_ptr, "vals": sz.vals, "codes": sz.codes, "scales": sz.scales,
            "workspace": sz.workspace}


@dataclass
class PackedWeight:
    """A packed layer: four caller-owned device tensors plus the C descriptor."""
    rows: int
    cols: int
    n_keep: int
    group_size: int
    row_ptr: object          # torch.int32 [rows+1]
    vals: object             # torch.uint8 [nnz/2]
    codes: Optional[object]  # torch.int16 [nnz/8] (uint16 bits) or None
    scales: object           # torch.int16 [rows*cols/G] (fp16 bits)
    sse: Dict[int, int] = field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return self.rows * self.cols * self.n_keep // 4

    def descriptor(self) -> B.i4s_packed:
        d = B.i4s_packed()
        d.rows, d.cols, d.n_keep, d.group_size = self.rows, self.cols, self.n_keep, self.group_size
        d.nnz = self.nnz
        d.row_ptr = self.row_ptr.data_ptr()
        d.vals = self.vals.data_ptr()
        d.codes = self.codes.data_ptr() if self.codes is not None else None
        n_scales = self.rows * (self.cols // self.group_size)
        d.scales = self.scales.data_ptr()
        assert self.scales.numel() >= n_scales
        return d

    def packed_nbytes(self) -> int:
        """Bytes one GEMV call must read: vals + codes + scales in use + row_ptr."""
        codes = self.nnz // 4 if self.n_keep < 4 else 0
        return self.nnz // 2 + codes + 2 * self.rows * (self.cols // self.group_size) + 4 * (self.rows + 1)


def pack(w, n_keep: int = 2, group_size: int = 128, col_norm=None, grad=None) -> PackedWeight:
    """Pack a [rows][cols] fp16 CUDA tensor.  group_size 0 chooses G per matrix.

    ``col_norm`` (float32 [cols], the activation norms ||X_j||_2) and
    ``grad`` (float16 [rows][cols], dE/dW) are the optional inputs of the
    Eq. (3) importance score (``i4s_pack_ex``); without them the mask is by
    magnitude (``i4s_pack``).
    """
    torch = _torch()
    if w.dtype != torch.float16 or w.dim() != 2 or not w.is_cuda:
        raise ValueError("w must be a 2-D float16 tensor on a GPU")
    w = w.contiguous()
    rows, cols = w.shape
    if col_norm is not None:
        if col_norm.dtype != torch.float32 or tuple(col_norm.shape) != (cols,) or col_norm.device != w.device:
            raise ValueError("col_norm must be a float32 [cols] tensor on w's device")
        col_norm = col_norm.contiguous()
    if grad is not None:
        if grad.dtype != torch.float16 or tuple(grad.shape) != (rows, cols) or grad.device != w.device:
            raise ValueError("grad must be a float16 tensor of w's shape on w's device")
        grad = grad.contiguous()
    sz = pack_sizes(rows, cols, n_keep, group_size)
    dev = w.device
    row_ptr = torch.empty(sz["row_ptr"] // 4, dtype=torch.int32, device=dev)
    vals = torch.empty(sz["vals"], dtype=torch.uint8, device=dev)
    codes = torch.empty(sz["codes"] // 2, dtype=torch.int16, device=dev) if n_keep < 4 else None
    scales = torch.empty(sz["scales"] // 2, dtype=torch.int16, device=dev)
    ws = torch.empty(sz["workspace"], dtype=torch.uint8, device=dev)
    d = B.i4s_packed()
    d.row_ptr, d.vals = row_ptr.data_ptr(), vals.data_ptr()
    d.codes = codes.data_ptr() if codes is not None else None
    d.scales = scales.data_ptr()
    rep = B.i4s_pack_report()
    with torch.cuda.device(dev):
        if col_norm is None and grad is None:
            st = B.i4s_pack(w.data_ptr(), rows, cols, n_keep, group_size, ws.data_ptr(), sz["workspace"],
                            d, rep, _stream_handle(dev))
        else:
            st = B.i4s_pack_ex(w.data_ptr(), rows, cols, n_keep, group_size,
                               col_norm.data_ptr() if col_norm is not None else None,
                               grad.data_ptr() if grad is not None else None,
                               ws.data_ptr(), sz["workspace"], d, rep, _stream_handle(dev))
    B.check(st, "i4s_pack")
    g = d.group_size
    scales = scales[: rows * (cols // g)]
    sse = {}
    if rep.n_candidates:
        for i in range(3):
            sse[rep.candidates[i]] = (int(rep.sse_hi[i]) << 64) | int(rep.sse_lo[i])
    del ws  # freed only after the stream has used it: torch's caching allocator is stream-ordered
    return PackedWeight(rows, cols, n_keep, g, row_ptr, vals, codes, scales, sse)


def run_workspace_size(p: PackedWeight, batch: int) -> int:
    n = ctypes.c_uint64()
    B.check(B.i4s_run_workspace_size(p.descriptor(), batch, n), "i4s_run_workspace_size")
    return n.value


# One scratch workspace per (device, stream), grown on demand.  Calls on one
# stream are ordered, so they can share it.
_WORKSPACES: Dict[tuple, object] = {}


def _workspace(device, stream_handle: int, nbytes: int):
    torch = _torch()
    key = (device.index, stream_handle)
    t = _WORKSPACES.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WORKSPACES[key] = t
    return t


def _check_out(out, batch: int, rows: int, device) -> None:
    torch = _torch()
    if (out.dtype != torch.float16 or tuple(out.shape) != (batch, rows) or out.device != device
            or not out.is_contiguous()):
        raise ValueError(f"out must be a contiguous float16 [{batch}][{rows}] tensor on {device}")


def run(p: PackedWeight, x, out=None, descriptor: Optional[B.i4s_packed] = None, workspace=None,
        use_workspace: bool = True):
    """y = W_hat x for x of shape [batch][cols] (or [cols]) fp16 on the GPU.

    With ``use_workspace`` (the default) calls that can use one go through
    ``i4s_run_ws`` with ``workspace`` (a uint8 device tensor of at least
    ``run_workspace_size`` bytes) or a cached per-stream workspace; otherwise
    through ``i4s_run``.
    """
    torch = _torch()
    squeeze = x.dim() == 1
    if squeeze:
        x = x.unsqueeze(0)
    if x.dtype != torch.float16 or x.dim() != 2 or x.shape[1] != p.cols or not x.is_cuda:
        raise ValueError("x must be float16 [batch][cols] on the GPU")
    if p.vals.device != x.device:
        raise ValueError(f"x is on {x.device}, the packed layer on {p.vals.device}")
    x = x.contiguous()
    batch = x.shape[0]
    if out is None:
        out = torch.empty(batch, p.rows, dtype=torch.float16, device=x.device)
    else:
        _check_out(out, batch, p.rows, x.device)
    d = descriptor if descriptor is not None else p.descriptor()
    stream = _stream_handle(x.device)
    nbytes = 0
    if use_workspace:
        n = ctypes.c_uint64()
        B.check(B.i4s_run_workspace_size(d, batch, n), "i4s_run_workspace_size")
        nbytes = n.value
    if nbytes:
        ws = workspace if workspace is not None else _workspace(x.device, stream, nbytes)
        if ws.device != x.device or not ws.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on x's device")
        B.check(B.i4s_run_ws(d, x.data_ptr(), batch, out.data_ptr(), ws.data_ptr(),
                             ws.numel() * ws.element_size(), stream), "i4s_run_ws")
    else:
        B.check(B.i4s_run(d, x.data_ptr(), batch, out.data_ptr(), stream), "i4s_run")
    return out[0] if squeeze else out


def run_multi(layers, x, outs=None):
    """y_m = W_hat_m x for layers sharing x, in one launch where possible.

    ``layers``: PackedWeight objects with the same cols.  ``x``: float16
    [batch][cols] (or [cols]) on the GPU.  Returns a list of outputs (or
    fills ``outs``).  Calls ``i4s_run_multi``.
    """
    torch = _torch()
    squeeze = x.dim() == 1
    if squeeze:
        x = x.unsqueeze(0)
    if x.dtype != torch.float16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be float16 [batch][cols] on the GPU")
    for p in layers:
        if p.vals.device != x.device:
            raise ValueError(f"x is on {x.device}, a packed layer on {p.vals.device}")
    x = x.contiguous()
    batch = x.shape[0]
    if outs is None:
        outs = [torch.empty(batch, p.rows, dtype=torch.float16, device=x.device) for p in layers]
    else:
        if len(outs) != len(layers):
            raise ValueError(f"{len(outs)} outputs for {len(layers)} layers")
        for o, p in zip(outs, layers):
            _check_out(o, batch, p.rows, x.device)
    descs = [p.descriptor() for p in layers]
    B.check(B.i4s_run_multi(descs, x.data_ptr(), batch, [o.data_ptr() for o in outs], _stream_handle(x.device)),
            "i4s_run_multi")
    return [o[0] for o in outs] if squeeze else outs
