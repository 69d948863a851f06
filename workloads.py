"""Seeded synthetic inputs for the INT4 2-bit-CSR SparseGEMV.

This module only draws random numbers and names shapes. It holds none of the
method's arithmetic (no masking, scaling, quantization, packing or GEMV), so
both the CPU oracle side and the HIP side of the tests and the benchmark can
take their inputs from here without sharing any computation.

Recipe (one numpy ``default_rng(seed)`` stream per matrix):

* W: ``0.02 * standard_normal((R, K))`` in float64.  When a workload asks for
  outliers, exactly ``round(0.01 * R * K)`` distinct flat positions drawn with
  ``rng.choice(R*K, n, replace=False)`` are multiplied by 8.  The result is
  rounded once to fp16 (round-to-nearest-even).
* x: drawn from the same stream after W, ``standard_normal((B, K))`` rounded to
  fp16.  W is therefore identical for every batch size B of a given seed.
* The largest layer of the tests (``make_weight_on_device``) is drawn on the
  GPU by torch's seeded generator: float32 ``0.02 * randn`` rounded once to
  fp16.  The rows the test checks are copied back from that tensor, so the
  oracle and the library see the same weights.
* Importance inputs (``make_importance_inputs``, a stream of their own):
  column norms ``16 * exp(0.5 * standard_normal(K))`` in float32, with 1 % of
  the columns (at least one) set to 0 (dead channels) and 1 % (at least one)
  multiplied by 20 (outlier channels); gradients ``1e-3 *
  standard_normal((R, K))`` rounded to fp16.  The tie-heavy variant draws
  norms from {0, 0.5, 1, 2} and gradients from {0, +-0.25, +-1} so that many
  scores coincide exactly.

The shapes stand in for the decoder layers of a 7B-class and a 13B-class
model; the page this work follows measures a 1.5B model on proprietary and
public data that are not used here.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

__all__ = ["Matrix", "Workload", "WORKLOADS", "make_weight", "make_x",
           "make_weight_and_x", "make_importance_inputs", "stack_7b_matrices"]


@dataclass(frozen=True)
class Matrix:
    """One weight matrix of a workload: rows R (out features) x cols K (in features)."""
    name: str
    rows: int
    cols: int
    n_keep: int          # 2 for 2:4, 4 for dense INT4, 1 for 1:4
    group_size: int      # 64/128/256, or 0 for "choose per matrix by minimum MSE"
    seed: int
    outliers: bool = False


@dataclass(frozen=True)
class Workload:
    name: str
    matrices: Tuple[Matrix, ...]
    batches: Tuple[int, ...]
    description: str = ""


def make_weight(rows: int, cols: int, seed: int, outliers: bool = False,
                rng: Optional[np.random.Generator] = None) -> np.ndarray:
    """fp16 weight [rows][cols], N(0, 0.02^2), optional 1 % outliers x8."""
    if rng is None:
        rng = np.random.default_rng(seed)
    w = 0.02 * rng.standard_normal((rows, cols))
    if outliers:
        n = int(round(0.01 * rows * cols))
        idx = rng.choice(rows * cols, n, replace=False)
        w.reshape(-1)[idx] *= 8.0
    return w.astype(np.float16)


def make_weight_on_device(rows: int, cols: int, seed: int, device):
    """fp16 weight [rows][cols], N(0, 0.02^2), drawn on ``device`` by torch's
    seeded generator for that device (float32 normals, times 0.02, rounded
    once to fp16): a layer of several GB without a host copy.  Only the test
    of the largest layer uses it; the rows it checks are read back from the
    returned tensor."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    w = torch.empty((rows, cols), dtype=torch.float16, device=device)
    step = max(1, (1 << 26) // cols)  # 256 MiB of float32 at a time
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        w[r0:r1] = (0.02 * torch.randn((r1 - r0, cols), generator=g, device=device, dtype=torch.float32)).half()
    return w


def make_x(rng: np.random.Generator, batch: int, cols: int) -> np.ndarray:
    """fp16 activations [batch][cols], N(0, 1)."""
    return rng.standard_normal((batch, cols)).astype(np.float16)


def make_weight_and_x(m: Matrix, batch: int) -> Tuple[np.ndarray, np.ndarray]:
    """W for matrix ``m`` and x for ``batch`` vectors, from one seeded stream."""
    rng = np.random.default_rng(m.seed)
    w = make_weight(m.rows, m.cols, m.seed, m.outliers, rng=rng)
    x = make_x(rng, batch, m.cols)
    return w, x


def make_importance_inputs(rows: int, cols: int, seed: int,
                           tie_heavy: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """(column norms float32 [cols], gradients fp16 [rows][cols])."""
    rng = np.random.default_rng(seed)
    if tie_heavy:
        norm = rng.choice(np.float32([0.0, 0.5, 1.0, 2.0]), cols)
        grad = rng.choice(np.float16([0.0, 0.25, -0.25, 1.0, -1.0]), (rows, cols))
        return norm.astype(np.float32), grad.astype(np.float16)
    norm = 16.0 * np.exp(0.5 * rng.standard_normal(cols))
    n = max(1, int(round(0.01 * cols)))
    idx = rng.choice(cols, 2 * n, replace=False)
    norm[idx[:n]] = 0.0
    norm[idx[n:]] *= 20.0
    grad = 1e-3 * rng.standard_normal((rows, cols))
    return norm.astype(np.float32), grad.astype(np.float16)


_PROJ = ("q", "k", "v", "o", "gate", "up", "down")


def stack_7b_matrices(outer: int = 4, inner: int = 2) -> Tuple[Matrix, ...]:
    """The 224 projections of a 32-layer 7B-shaped decoder, in layer order.

    Layers 0-3 and 28-31 take pattern ``outer`` (n_keep; dense INT4 = 4 by
    default), the others ``inner`` (2:4 by default); each matrix picks its
    own group size; seed = 100 + 7*layer + projection index, so the weights
    are the same whatever the patterns.
    """
    out: List[Matrix] = []
    for layer in range(32):
        n_keep = outer if (layer < 4 or layer >= 28) else inner
        for m, proj in enumerate(_PROJ):
            if proj in ("q", "k", "v", "o"):
                r, k = 4096, 4096
            elif proj in ("gate", "up"):
                r, k = 11008, 4096
            else:
                r, k = 4096, 11008
            out.append(Matrix(f"L{layer}.{proj}", r, k, n_keep, 0, 100 + 7 * layer + m))
    return tuple(out)


WORKLOADS = {
    "c1_512": Workload(
        "c1_512", (Matrix("w", 512, 512, 2, 128, 0),), (1,),
        "single 512x512 layer, 2:4, G=128, batch 1"),
    "c2_4096": Workload(
        "c2_4096", (Matrix("w", 4096, 4096, 2, 128, 0),), (1,),
        "single 4096x4096 layer (7B attention projection), 2:4, G=128, batch 1"),
    "c3_mlp7b": Workload(
        "c3_mlp7b",
        (Matrix("up", 11008, 4096, 2, 0, 0, True),
         Matrix("gate", 11008, 4096, 2, 0, 1, True),
         Matrix("down", 4096, 11008, 2, 0, 2, True)),
        (1,),
        "7B MLP projections with 1% x8 outliers, 2:4, adaptive G, batch 1"),
    "c4_stack7b": Workload(
        "c4_stack7b", stack_7b_matrices(), (1,),
        "32-layer 7B stack, dense INT4 in layers 0-3/28-31, 2:4 elsewhere, adaptive G, batch 1"),
    "c5_verify13b": Workload(
        "c5_verify13b",
        (Matrix("attn", 5120, 5120, 2, 128, 0),
         Matrix("up", 13824, 5120, 2, 128, 1),
         Matrix("down", 5120, 13824, 2, 128, 2)),
        (4, 8, 16),
        "13B-shaped layers, 2:4, G=128, verification batches of 4, 8 and 16"),
    # the 1:4 pattern and the layer-wise 2:4/1:4 mix of the page's
    # "Sparse(Mix)+Quant" setting (which layers count as critical is not
    # given; here the outer four at each end keep 2:4)
    "x1_4096_1to4": Workload(
        "x1_4096_1to4", (Matrix("w", 4096, 4096, 1, 128, 0),), (1, 4, 8, 16),
        "single 4096x4096 layer, 1:4, G=128, batches 1, 4, 8 and 16"),
    "x2_mix_stack7b": Workload(
        "x2_mix_stack7b", stack_7b_matrices(outer=2, inner=1), (1,),
        "32-layer 7B stack, 2:4 in layers 0-3/28-31, 1:4 elsewhere, adaptive G, batch 1"),
}
