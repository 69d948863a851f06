"""Build libi4s.so in-tree with hipcc for gfx950.

``python -m int4_sparse_gemv_amd.build`` (or ``build()``) compiles the
library's HIP and C++ sources under ``csrc/`` into
``int4_sparse_gemv_amd/libi4s.so``, and the benchmark's floor kernels
(``csrc/i4s_floor.hip``) into ``libi4s_floor.so``.  It always recompiles.
hipcc cross-compiles for gfx950 without a GPU present.

``--define NAME=VALUE`` (repeatable) overrides one of the kernel-choice
thresholds of ``csrc/i4s_internal.h`` and ``--out PATH`` writes that build of
the library elsewhere (for measuring the alternatives with ``bench.py
--lib PATH``); the default library is only ever built with the defaults.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libi4s.so")
FLOOR_LIB = os.path.join(PKG, "libi4s_floor.so")

SOURCES = ("i4s_api.cpp", "i4s_plan.cpp", "i4s_pack.hip", "i4s_gemv_b1.hip", "i4s_gemv_b2.hip", "i4s_gemv_batch.hip",
           "i4s_noalloc.hip")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # IEEE-correct fp32 division (the packer's scale and quantizer rely on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # keep packed-fp32 VALU forms out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 16 kernel-argument dwords arrive in SGPRs at wave start, so
    # the GEMV's first loads do not wait for a scalar memory round trip (the
    # code object keeps a fallback that loads them itself)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    # matrix instructions read and write their accumulators in VGPRs: left to
    # its heuristics the compiler put the K-split kernel's per-group tiles in
    # AGPRs, and every group then cost 4 v_accvgpr_read + 4 v_accvgpr_write
    # (8 of ~26 VALU instructions per unit); the other kernels already used
    # VGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libi4s)")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _compile(cc, src, tmp, defines=()):
    obj = os.path.join(tmp, src + ".o")
    cmd = [cc, *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", INCLUDE, "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", obj]
    return obj, _run(cmd)


def _link(cc, sources, lib, tmp, verbose, defines=()):
    # one hipcc process per source, in parallel (the batch kernels dominate)
    jobs = max(1, min(len(sources), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        done = list(ex.map(lambda src: _compile(cc, src, tmp, defines), sources))
    objs = []
    for obj, out in done:
        if verbose and out.strip():
            print(out)
        objs.append(obj)
    tmp_lib = lib + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib])
    os.replace(tmp_lib, lib)


THRESHOLDS = ("I4S_BATCH2_VALU_MAX_ROWS", "I4S_BATCH2_VALU_MAX_K", "I4S_MATRIX_CORE_MIN_BATCH")


def build(verbose: bool = False, defines=(), out: str = None) -> str:
    """Compile libi4s.so and libi4s_floor.so; returns the path of libi4s.so.

    With ``defines`` (NAME=VALUE strings, NAME one of THRESHOLDS) and ``out``,
    build only the library, with those thresholds, at ``out``."""
    for d in defines:
        if d.split("=", 1)[0] not in THRESHOLDS or "=" not in d:
            raise ValueError(f"--define takes NAME=VALUE with NAME in {THRESHOLDS}, got {d!r}")
    if defines and not out:
        raise ValueError("a build with --define needs --out (the default library keeps the defaults)")
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="i4s_build_") as tmp:
        if out:
            os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
            _link(cc, SOURCES, os.path.abspath(out), tmp, verbose, tuple(defines))
            return os.path.abspath(out)
        _link(cc, SOURCES, LIB, tmp, verbose)
        _link(cc, ("i4s_floor.hip",), FLOOR_LIB, tmp, verbose)
    return LIB


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("--define", action="append", default=[])
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    print(build(verbose=a.v, defines=a.define, out=a.out))
