"""Write the oracle's digests of every matrix of the two 32-layer stacks.

Calls only the CPU oracle (``oracle/``) and the seeded generators
(``workloads.py``).  For each of the 224 matrices of the dense/2:4 stack and
the 224 of the mixed 2:4/1:4 stack it packs the seeded fp16 weight with the
adaptive group size (the oracle's exact-SSE argmin over {64, 128, 256}) and
records the chosen G, the three exact SSEs (units of 2^-48, as decimal
strings) and the SHA-256 of each packed buffer (row_ptr as little-endian
int32, vals as bytes, codes and scales as little-endian uint16).

The GPU stack test compares the library's pack of the same weights with
these records, and recomputes the oracle's GEMV reference at the recorded G
on the CPU at test time (the reference outputs are too large to store).

Rules followed (section 3.1 and 3.2 of "Efficient LLM-based Advertising via
Model Compression and Parallel Verification": layer-wise N:M sparsity and
group-wise INT4 quantization with a per-layer group size; section 3.3: the
2-bit CSR buffers).

    python tests/golden/make_stack_digests.py [--jobs N]

takes about an hour of CPU time (a few minutes per core on 8 cores).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "stack_digests.json")
STACKS = ("c4_stack7b", "x2_mix_stack7b")


def buffer_digests(packed) -> dict:
    import numpy as np
    as_bytes = {
        "row_ptr": np.asarray(packed["row_ptr"], dtype="<i4").tobytes(),
        "vals": np.asarray(packed["vals"], dtype=np.uint8).tobytes(),
        "codes": np.asarray(packed["codes"], dtype="<u2").tobytes(),
        "scales": np.asarray(packed["scales"], dtype="<u2").tobytes(),
    }
    return {k: hashlib.sha256(v).hexdigest() for k, v in as_bytes.items()}


def one(task):
    workload, index = task
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import oracle as O
    import workloads as WL
    m = WL.WORKLOADS[workload].matrices[index]
    w, _ = WL.make_weight_and_x(m, 1)
    ref = O.pack(w, m.n_keep, m.group_size)
    return {
        "workload": workload, "index": index, "name": m.name, "rows": m.rows, "cols": m.cols,
        "n_keep": m.n_keep, "seed": m.seed, "group_size": int(ref["group_size"]),
        "sse": {str(g): str(v) for g, v in sorted(ref["sse"].items())},
        "sha256": buffer_digests(ref),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(6, os.cpu_count() or 1))
    args = ap.parse_args()
    sys.path.insert(0, ROOT)
    import workloads as WL
    tasks = [(name, i) for name in STACKS for i in range(len(WL.WORKLOADS[name].matrices))]
    t0 = time.time()
    out = []
    with ProcessPoolExecutor(args.jobs, mp_context=mp.get_context("spawn")) as ex:
        for k, rec in enumerate(ex.map(one, tasks)):
            out.append(rec)
            print(f"{k + 1}/{len(tasks)} {rec['workload']}/{rec['name']} G{rec['group_size']} "
                  f"{time.time() - t0:.0f} s", flush=True)
    with open(OUT, "w") as f:
        json.dump({"generator": "tests/golden/make_stack_digests.py (oracle/ and workloads.py only)",
                   "matrices": out}, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
