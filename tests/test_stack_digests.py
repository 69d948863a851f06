"""The stored oracle digests of the two 32-layer stacks match the oracle (CPU).

``golden/stack_digests.json`` is written by ``golden/make_stack_digests.py``
from the oracle alone; the GPU stack test compares the library against it.
Here a sample of its records is recomputed with the oracle, and the file is
checked to list every matrix of both stacks with the workload's shapes,
patterns and seeds.
"""

import json
import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

import oracle as O  # noqa: E402
import stack_oracle_worker as SW  # noqa: E402
import workloads as WL  # noqa: E402

DIGESTS = os.path.join(HERE, "golden", "stack_digests.json")


def load():
    with open(DIGESTS) as f:
        return {(m["workload"], m["index"]): m for m in json.load(f)["matrices"]}


def test_digest_file_lists_every_stack_matrix():
    rec = load()
    assert len(rec) == 2 * 224
    for name in SW.STACKS:
        for i, m in enumerate(WL.WORKLOADS[name].matrices):
            r = rec[(name, i)]
            assert (r["name"], r["rows"], r["cols"], r["n_keep"], r["seed"]) == (m.name, m.rows, m.cols, m.n_keep, m.seed)
            assert r["group_size"] in (64, 128, 256)
            sse = {int(g): int(v) for g, v in r["sse"].items()}
            assert sorted(sse) == [64, 128, 256]
            # the recorded G is the argmin, ties going to the larger group
            best = min(sse.values())
            assert r["group_size"] == max(g for g, v in sse.items() if v == best)
            assert all(len(h) == 64 for h in r["sha256"].values())


@pytest.mark.parametrize("index", [28, 31])  # L4.q (2:4 and 1:4) and L4.o
def test_digest_records_match_the_oracle(index):
    rec = load()
    for name in SW.STACKS:
        m = WL.WORKLOADS[name].matrices[index]
        w, _ = WL.make_weight_and_x(m, 1)
        ref = O.pack(w, m.n_keep, m.group_size)
        r = rec[(name, index)]
        assert ref["group_size"] == r["group_size"]
        assert {str(g): str(v) for g, v in ref["sse"].items()} == r["sse"]
        assert SW.buffer_digests(ref) == r["sha256"]
