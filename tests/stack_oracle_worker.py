"""CPU side of the stack parity test: the oracle's reference for one seed.

Runs in worker processes started with the ``spawn`` method (never forked
from a process that has touched the GPU) and imports only NumPy, the oracle
and the seeded generators -- no torch, no library code.

For matrix ``index`` of the 32-layer stacks it draws the seeded fp16 weight
and the batch-1 activation vector (both stacks use the same seed, shape and
therefore the same W and x for a given index), then for each stack packs W
with the oracle at the group size recorded by ``golden/make_stack_digests.py``
and returns the SHA-256 of the packed buffers and the oracle's GEMV reference
y_ref = W_hat x and a_ref = |W_hat| |x| in float64.
"""

from __future__ import annotations

import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
STACKS = ("c4_stack7b", "x2_mix_stack7b")


def buffer_digests(packed) -> dict:
    """SHA-256 of row_ptr (little-endian int32), vals, codes and scales
    (little-endian uint16) -- the encoding the digest file records."""
    import numpy as np
    as_bytes = {
        "row_ptr": np.asarray(packed["row_ptr"], dtype="<i4").tobytes(),
        "vals": np.asarray(packed["vals"], dtype=np.uint8).tobytes(),
        "codes": np.asarray(packed["codes"], dtype="<u2").tobytes(),
        "scales": np.asarray(packed["scales"], dtype="<u2").tobytes(),
    }
    return {k: hashlib.sha256(v).hexdigest() for k, v in as_bytes.items()}


def reference(task):
    """task = (index, {stack name: recorded group size}) -> dict with W, x and,
    per stack, the oracle's buffer digests, y_ref and a_ref (batch 1)."""
    index, group_sizes = task
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import oracle as O
    import workloads as WL
    mats = {name: WL.WORKLOADS[name].matrices[index] for name in STACKS}
    first = mats[STACKS[0]]
    for m in mats.values():
        assert (m.rows, m.cols, m.seed, m.outliers) == (first.rows, first.cols, first.seed, first.outliers)
    w, x = WL.make_weight_and_x(first, 1)
    out = {"index": index, "w": w, "x": x}
    for name, m in mats.items():
        ref = O.pack(w, m.n_keep, group_sizes[name])
        y_ref, a_ref = O.run(ref, x)
        out[name] = {"sha256": buffer_digests(ref), "y_ref": y_ref, "a_ref": a_ref}
        del ref
    return out
