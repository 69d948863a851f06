"""GPU parity on every matrix of the two 32-layer 7B-shaped stacks (needs an MI355X).

448 matrices: the dense-INT4/2:4 stack (dense in layers 0-3 and 28-31) and the
mixed 2:4/1:4 stack (2:4 in those layers, 1:4 elsewhere), each matrix with its
own seed and an adaptively chosen group size (section 3.1 and 3.2 of
"Efficient LLM-based Advertising via Model Compression and Parallel
Verification": layer-wise N:M sparsity, group-wise INT4 with a per-layer
group size; section 3.3: the 2-bit CSR buffers and the SparseGemv).

For each matrix the library packs the seeded weight on the GPU with
group_size 0 (adaptive) and must
  * choose the group size and report the three exact SSEs that the oracle
    recorded in ``golden/stack_digests.json`` (written by
    ``golden/make_stack_digests.py``, which calls only the oracle and the
    seeded generators);
  * produce row_ptr, vals, codes and scales whose SHA-256 equal the recorded
    ones and those of the oracle's pack recomputed on the CPU in this run;
  * compute y at batch 1 within 1e-3 * sum_j |w_hat_ij x_j| + 1e-5 of the
    oracle's float64 reference, element by element.
The oracle side runs in CPU worker processes started with ``spawn`` (they
import neither torch nor the library) while the GPU side checks the
matrices in layer order.
"""

import hashlib
import json
import multiprocessing as mp
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

import stack_oracle_worker as SW  # noqa: E402
import workloads as WL  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DIGESTS = os.path.join(HERE, "golden", "stack_digests.json")
N_MATRICES = 224
PER_LAYER = 7


def say(msg):
    print(msg, flush=True)


def _records():
    with open(DIGESTS) as f:
        d = json.load(f)
    rec = {(m["workload"], m["index"]): m for m in d["matrices"]}
    for name in SW.STACKS:
        for i, m in enumerate(WL.WORKLOADS[name].matrices):
            r = rec[(name, i)]
            assert (r["name"], r["rows"], r["cols"], r["n_keep"], r["seed"]) == \
                   (m.name, m.rows, m.cols, m.n_keep, m.seed), f"digest record {name}/{i} is stale"
    return rec


class OracleFeed:
    """Oracle references for matrices 0..223, computed ahead by a pool of
    spawned CPU workers and handed out in layer order."""

    def __init__(self, rec):
        workers = max(1, min(12, len(os.sched_getaffinity(0)) - 1))
        tasks = [(i, {name: rec[(name, i)]["group_size"] for name in SW.STACKS}) for i in range(N_MATRICES)]
        self.pool = mp.get_context("spawn").Pool(workers)
        self.it = self.pool.imap(SW.reference, tasks, chunksize=1)
        self.done = {}
        self.next = 0
        say(f"stack oracle: {workers} CPU workers for {N_MATRICES} seeds")

    def get(self, index):
        while index not in self.done:
            r = self.it.next(timeout=600)
            self.done[r["index"]] = r
        return self.done.pop(index)

    def close(self):
        self.pool.terminate()
        self.pool.join()


@pytest.fixture(scope="module")
def feed():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_sparse_gemv_amd as I
    I._binding.load()  # raises if the library is not built
    f = OracleFeed(_records())
    yield f
    f.close()


@pytest.fixture(scope="module")
def records():
    return _records()


def gpu_digests(p):
    """SHA-256 of the library's packed buffers in the digest file's encoding."""
    codes = p.codes.cpu().numpy().view("<u2") if p.codes is not None else np.zeros(0, "<u2")
    as_bytes = {
        "row_ptr": p.row_ptr.cpu().numpy().astype("<i4").tobytes(),
        "vals": p.vals.cpu().numpy().astype(np.uint8).tobytes(),
        "codes": codes.tobytes(),
        "scales": p.scales.cpu().numpy().view("<u2").tobytes(),
    }
    return {k: hashlib.sha256(v).hexdigest() for k, v in as_bytes.items()}


@pytest.mark.parametrize("layer", range(N_MATRICES // PER_LAYER))
def test_stack_layer_pack_and_gemv(feed, records, layer):
    import int4_sparse_gemv_amd as I
    for index in range(PER_LAYER * layer, PER_LAYER * (layer + 1)):
        r = feed.get(index)
        w = torch.from_numpy(r["w"].view(np.int16)).cuda().view(torch.float16)
        x = torch.from_numpy(r["x"].view(np.int16)).cuda().view(torch.float16)
        for name in SW.STACKS:
            m = WL.WORKLOADS[name].matrices[index]
            rec = records[(name, index)]
            label = f"{name}/{m.name} {m.rows}x{m.cols} n={m.n_keep}"
            say(f"case stack {label}")
            p = I.pack(w, m.n_keep, m.group_size)
            y = I.run(p, x)
            torch.cuda.synchronize()
            assert p.group_size == rec["group_size"], f"{label}: G {p.group_size} != {rec['group_size']}"
            assert {str(g): str(v) for g, v in p.sse.items()} == rec["sse"], f"{label}: SSE {p.sse} != {rec['sse']}"
            got = gpu_digests(p)
            assert r[name]["sha256"] == rec["sha256"], f"{label}: the oracle's pack differs from its record"
            for k in ("row_ptr", "vals", "codes", "scales"):
                assert got[k] == rec["sha256"][k], f"{label}: {k} differs from the oracle's"
            y_gpu = y.cpu().numpy().astype(np.float64)
            err = np.abs(y_gpu - r[name]["y_ref"])
            tol = 1e-3 * r[name]["a_ref"] + 1e-5
            bad = np.argwhere(err > tol)
            assert bad.size == 0, (f"{label}: {len(bad)} outputs outside tolerance, first {bad[:3].tolist()}, "
                                   f"max err/tol {float((err / tol).max()):.3g}")
            del p, y
        del w, x, r
