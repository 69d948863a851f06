"""Benchmark of the packed INT4 2-bit-CSR SparseGEMV on one MI355X.

One step = one ``i4s_run_ws`` call (the whole per-call hot path: stage x, stream
the packed weights, decode, multiply-accumulate, reduce, store y) over one
batch of synthetic input.  The layer is packed once beforehand (packing is
offline work); its time is reported separately as ``pack_ms``.

Cold (the headline): the packed layer is copied P = ceil(1 GiB / packed
bytes) times (byte-identical device copies, > 4x the 256 MB last-level
cache) and the steps visit the copies round-robin, so every call streams its
weights from HBM.  Hot (reported, labelled cache-resident): one copy.  The K
timed steps are captured once into a HIP graph and replayed, so host launch
overhead does not pace the GPU; the graph holds exactly K launches.  The
timed replay is bracketed by torch.cuda.synchronize() and by HIP events on
the stream the kernels run on.

Prints ONE JSON line for the 4096x4096 2:4 G128 batch-1 layer.  ``value`` is
packed bytes per call / seconds per call (GB/s, decimal) in cold mode.
``--suite FILE`` additionally measures every workload (all matrices and
batch sizes, and the 224-call 7B stack in layer order) and writes a table.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD specification
METRIC = "µs/call and effective HBM GB/s (% of peak) of packed INT4 SparseGEMV, 4096×4096 b=1"
# the batch-1 kernel's sources: a traffic profile is used only while they are unchanged
B1_SRCS = [os.path.join(ROOT, "int4_sparse_gemv_amd", "csrc", f) for f in ("i4s_gemv_b1.hip", "i4s_gemv_common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_c2_4096.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c2_4096")
    ap.add_argument("--matrix", default=None, help="matrix name inside the workload (default: first)")
    ap.add_argument("--batch", type=int, default=None)
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (PMC traffic calibration)")
    ap.add_argument("--eager", action="store_true", help="time plain stream launches instead of a graph")
    ap.add_argument("--suite", default=None, help="also measure every workload and write a table here")
    ap.add_argument("--no-stack", action="store_true", help="with --suite: skip the 224-matrix 7B stack")
    ap.add_argument("--only", default=None, help="with --suite: comma-separated workloads to measure")
    ap.add_argument("--suite-steps", type=int, default=1000, help="with --suite: timed calls per layer and trial")
    ap.add_argument("--no-floors", action="store_true",
                    help="skip the read-only and latency floor measurements")
    return ap.parse_args()


def sha_of(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Runner:
    """Packs layers and times graph-captured sequences of i4s_run calls."""

    def __init__(self, args):
        import torch
        import int4_sparse_gemv_amd as I
        from int4_sparse_gemv_amd import _binding as B
        self.torch, self.I, self.B, self.args = torch, I, B, args
        self.lib = B.load()
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.stream = torch.cuda.current_stream(self.dev)
        self.keep = []

    def to_dev(self, a16):
        import numpy as np
        return self.torch.from_numpy(a16.view(np.int16)).to(self.dev).view(self.torch.float16)

    def pack(self, w16, m):
        """Returns (packed weight, pack milliseconds)."""
        torch = self.torch
        w = self.to_dev(w16)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        p = self.I.pack(w, m.n_keep, m.group_size)
        torch.cuda.synchronize()
        return p, (time.perf_counter() - t0) * 1e3

    def clone(self, p):
        return self.I.PackedWeight(p.rows, p.cols, p.n_keep, p.group_size, p.row_ptr.clone(), p.vals.clone(),
                                   p.codes.clone() if p.codes is not None else None, p.scales.clone())

    def calls(self, items):
        """items: list of (packed, x tensor, y tensor, batch) -> list of i4s_run_ws argument tuples.

        Calls that can use a workspace share one scratch buffer (they run in
        order on one stream)."""
        out, need = [], 0
        for p, x, y, b in items:
            d = p.descriptor()
            self.keep.append(d)
            n = ctypes.c_uint64()
            self.B.check(self.B.i4s_run_workspace_size(d, b, n), "i4s_run_workspace_size")
            need = max(need, n.value)
            out.append([ctypes.byref(d), x.data_ptr(), b, y.data_ptr(), n.value])
        ws = self.torch.empty(max(need, 256), dtype=self.torch.uint8, device=self.dev)
        self.keep.append(ws)
        return [(d, xp, b, yp, ws.data_ptr() if n else None, ws.numel()) for d, xp, b, yp, n in out]

    def timed(self, seq, steps, warmup, trials):
        """Median (wall ms per step, event ms per step) over trials; seq is visited round-robin.

        An item of seq is an i4s_run_ws argument tuple or a callable taking
        the stream handle and returning a status."""
        import numpy as np
        torch, run_ws = self.torch, self.lib.i4s_run_ws

        def run(item, sh):
            return item(sh) if callable(item) else run_ws(*item, sh)
        walls, evs = [], []
        if self.args.eager:
            sh = self.stream.cuda_stream
            for i in range(warmup):
                assert run(seq[i % len(seq)], sh) == 0
            for _ in range(trials):
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                t = time.perf_counter()
                e0.record(self.stream)
                for i in range(steps):
                    run(seq[i % len(seq)], sh)
                e1.record(self.stream)
                torch.cuda.synchronize()
                walls.append((time.perf_counter() - t) * 1e3 / steps)
                evs.append(e0.elapsed_time(e1) / steps)
            return float(np.median(walls)), float(np.median(evs))
        cap = torch.cuda.Stream(self.dev)
        graphs = []
        for n in (warmup, steps):
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cap):
                for i in range(n):
                    st = run(seq[i % len(seq)], cap.cuda_stream)
                    if st != 0:
                        raise self.B.I4SError(st, "i4s_run")
            graphs.append(g)
        g_warm, g = graphs
        for _ in range(trials):
            g_warm.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t = time.perf_counter()
            e0.record(self.stream)
            g.replay()
            e1.record(self.stream)
            torch.cuda.synchronize()
            walls.append((time.perf_counter() - t) * 1e3 / steps)
            evs.append(e0.elapsed_time(e1) / steps)
        del graphs, g, g_warm
        return float(np.median(walls)), float(np.median(evs))

    def launch_floor_us(self, steps=2000):
        """Per-launch time of a one-element fill kernel replayed the same way (the dispatch floor)."""
        import numpy as np
        torch = self.torch
        t = torch.zeros(1, device=self.dev)
        cap = torch.cuda.Stream(self.dev)
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            for _ in range(steps):
                t.fill_(1.0)
        res = []
        for _ in range(3):
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            g.replay()
            e1.record(self.stream)
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) * 1e3 / steps)
        return float(np.median(res))

    def floors(self, nbytes, steps=2000, trials=3):
        """What one launch can reach at this size on this part, timed like the GEMV.

        stream_read_*: a kernel that only reads nbytes once (libi4s_floor.so,
        one 16-byte load per lane), cold over >= 1.5 GB of copies and hot;
        load_latency_ns: one lane chasing 4000 dependent loads through a random
        cycle spread over 2 GiB (one entry per KiB)."""
        import numpy as np
        from int4_sparse_gemv_amd import build as BLD
        torch = self.torch
        lib = ctypes.CDLL(BLD.FLOOR_LIB)
        lib.i4sf_stream_read.restype = ctypes.c_int
        lib.i4sf_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p]
        lib.i4sf_chase.restype = ctypes.c_int
        lib.i4sf_chase.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p]
        nb = nbytes // 16 * 16
        sink = torch.zeros(16, dtype=torch.int32, device=self.dev)
        copies = max(4, math.ceil(1.5 * (1 << 30) / nb))
        bufs = [torch.full((nb,), 0x5A, dtype=torch.uint8, device=self.dev) for _ in range(copies)]

        def timed_reads(nbuf, nt):
            cap = torch.cuda.Stream(self.dev)
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cap):
                for i in range(steps):
                    st = lib.i4sf_stream_read(bufs[i % nbuf].data_ptr(), nb, nt, sink.data_ptr(), cap.cuda_stream)
                    if st != 0:
                        raise RuntimeError(f"i4sf_stream_read returned {st}")
            res = []
            for _ in range(trials):
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(self.stream)
                g.replay()
                e1.record(self.stream)
                torch.cuda.synchronize()
                res.append(e0.elapsed_time(e1) * 1e3 / steps)
            del g
            return float(np.median(res))

        out = {"bytes": nb, "copies": copies,
               "stream_read_cold_us": {"nontemporal": timed_reads(copies, 1), "plain": timed_reads(copies, 0)},
               "stream_read_hot_us": timed_reads(1, 0)}
        del bufs
        # pointer chase: a single random cycle through M entries 1 KiB apart
        M, spacing, hops = 1 << 21, 256, 4000
        gen = torch.Generator(device=self.dev)
        gen.manual_seed(0)
        order = torch.randperm(M, device=self.dev, generator=gen, dtype=torch.int64)
        nxt = torch.zeros(M * spacing, dtype=torch.int32, device=self.dev)
        nxt[order * spacing] = (torch.roll(order, -1) * spacing).to(torch.int32)
        outv = torch.zeros(1, dtype=torch.int32, device=self.dev)
        lat = []
        for _ in range(trials):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            st = lib.i4sf_chase(nxt.data_ptr(), nxt.numel(), hops, outv.data_ptr(), self.stream.cuda_stream)
            e1.record(self.stream)
            torch.cuda.synchronize()
            if st != 0:
                raise RuntimeError(f"i4sf_chase returned {st}")
            lat.append(e0.elapsed_time(e1) * 1e6 / hops)
        k0 = int((order == 0).nonzero()[0])
        expect = int(order[(k0 + hops) % M]) * spacing
        if int(outv.item()) != expect:
            raise RuntimeError(f"pointer chase ended at {int(outv.item())}, expected {expect}")
        out["load_latency_ns"] = float(np.median(lat))
        del nxt, order
        torch.cuda.empty_cache()
        return out

    def measure_layer(self, m, batch, steps, warmup, trials):
        """Cold and hot timing of one matrix at one batch size."""
        import workloads as WL
        torch = self.torch
        w16, x16 = WL.make_weight_and_x(m, batch)
        p, pack_ms = self.pack(w16, m)
        x = self.to_dev(x16)
        y = torch.empty(batch, m.rows, dtype=torch.float16, device=self.dev)
        nbytes = p.packed_nbytes()
        n_cold = max(1, math.ceil((1 << 30) / nbytes))
        cps = [p] + [self.clone(p) for _ in range(n_cold - 1)]
        seq = self.calls([(c, x, y, batch) for c in cps])
        cold_wall, cold_ev = self.timed(seq, steps, warmup, trials)
        hot_wall, hot_ev = self.timed(seq[:1], steps, warmup, trials)
        del cps, seq
        self.keep.clear()
        torch.cuda.empty_cache()
        flops = 2 * (p.nnz) * batch
        return {"matrix": m.name, "rows": m.rows, "cols": m.cols, "n_keep": m.n_keep, "group_size": p.group_size,
                "batch": batch, "packed_bytes": nbytes, "copies": n_cold, "pack_ms": round(pack_ms, 3),
                "cold_wall_ms": cold_wall, "cold_us": cold_ev * 1e3, "hot_us": hot_ev * 1e3,
                "cold_gbs": nbytes / (cold_ev * 1e-3) / 1e9, "hot_gbs": nbytes / (hot_ev * 1e-3) / 1e9,
                "cold_tflops": flops / (cold_ev * 1e-3) / 1e12}

    def measure_stack(self, trials, name="c4_stack7b", fused=False):
        """The 224 projections of a 32-layer 7B stack in layer order: one call
        each, or (fused) q/k/v and gate/up as one i4s_run_multi call each, so
        4 calls per layer.  Fused projections read the same x, as in a model."""
        import workloads as WL
        torch = self.torch
        mats = WL.WORKLOADS[name].matrices
        items, total, groups = [], 0, {}
        for m in mats:
            w16, x16 = WL.make_weight_and_x(m, 1)
            p, _ = self.pack(w16, m)
            x = self.to_dev(x16)
            y = torch.empty(1, m.rows, dtype=torch.float16, device=self.dev)
            items.append((p, x, y, 1))
            total += p.packed_nbytes()
            groups[p.group_size] = groups.get(p.group_size, 0) + 1
        if fused:
            seq = []
            for layer in range(len(items) // 7):
                li = items[7 * layer: 7 * layer + 7]  # q, k, v, o, gate, up, down
                for grp in (li[0:3], li[3:4], li[4:6], li[6:7]):
                    if len(grp) == 1:
                        seq.extend(self.calls(grp))
                        continue
                    descs = [p.descriptor() for p, _, _, _ in grp]
                    arr = (self.B.i4s_packed * len(grp))(*descs)
                    ys = (ctypes.c_void_p * len(grp))(*[y.data_ptr() for _, _, y, _ in grp])
                    self.keep.extend([descs, arr, ys])
                    xp = grp[0][1].data_ptr()  # the group shares its first projection's x
                    seq.append(lambda sh, arr=arr, n=len(grp), xp=xp, ys=ys:
                               self.lib.i4s_run_multi(arr, n, xp, 1, ys, sh))
        else:
            seq = self.calls(items)
        wall, ev = self.timed(seq, len(seq), len(seq), trials)
        res = {"calls": len(seq), "fused": fused, "packed_bytes": total, "us_per_pass": ev * len(seq) * 1e3,
               "us_per_layer": ev * len(seq) * 1e3 / 32, "gbs": total / (ev * len(seq) * 1e-3) / 1e9,
               "group_sizes": groups}
        del items, seq
        self.keep.clear()
        torch.cuda.empty_cache()
        return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import workloads as WL

    R = Runner(args)
    wl = WL.WORKLOADS[args.workload]
    m = wl.matrices[0] if args.matrix is None else next(mm for mm in wl.matrices if mm.name == args.matrix)
    batch = args.batch or wl.batches[0]

    head = R.measure_layer(m, batch, args.steps, args.warmup, args.trials)
    floor_us = R.launch_floor_us()

    if args.calib_copy:
        torch = R.torch
        a = torch.empty(1 << 28, dtype=torch.uint8, device=R.dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    nbytes = head["packed_bytes"]
    achieved = nbytes / (head["cold_us"] * 1e-6) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("kernel_source_sha") == sha_of(B1_SRCS) and tr.get("workload") == args.workload
                and tr.get("batch") == batch):
            traffic = tr.get("hbm_bytes_per_launch")
    kname = kernel_label(m, batch)

    result = {
        "metric": METRIC,
        "value": round(nbytes / (head["cold_wall_ms"] * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["cold_wall_ms"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}/{m.name}: {m.rows}x{m.cols} "
                        f"{'dense' if m.n_keep == 4 else str(m.n_keep) + ':4'} INT4 G{head['group_size']}, "
                        f"batch {batch}, fp16 activations, fp32 accumulation",
            "rows": m.rows, "cols": m.cols, "n_keep": m.n_keep, "group_size": head["group_size"], "batch": batch,
            "mode": "cold", "copies": head["copies"], "timing": "eager" if args.eager else "hip_graph",
            "packed_bytes": nbytes, "x_bytes": 2 * batch * m.cols, "y_bytes": 2 * batch * m.rows,
        },
        "us_per_call": round(head["cold_us"], 4),
        "pct_of_peak": round(100 * achieved / PEAK_HBM_GBS, 2),
        "hot": {"us_per_call": round(head["hot_us"], 4), "gbs": round(head["hot_gbs"], 2),
                "note": "one copy, cache-resident (L2/MALL), not an HBM figure"},
        "launch_floor_us": round(floor_us, 4),
        "pack_ms": head["pack_ms"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": kname,
                     "algorithmic_bytes_per_launch": nbytes},
    }

    if not args.no_floors:
        fl = R.floors(nbytes)
        best = min(fl["stream_read_cold_us"].values())
        fl["read_only_ceiling_gbs"] = round(nbytes / (best * 1e-6) / 1e9, 2)
        fl["gemv_frac_of_read_only_ceiling"] = round(achieved / fl["read_only_ceiling_gbs"], 4)
        fl["empty_launch_us"] = round(floor_us, 4)
        for k in ("stream_read_hot_us", "load_latency_ns"):
            fl[k] = round(fl[k], 4)
        fl["stream_read_cold_us"] = {k: round(v, 4) for k, v in fl["stream_read_cold_us"].items()}
        result["floors"] = fl

    if args.suite:
        rows = run_suite(R, args)
        with open(args.suite, "w") as f:
            json.dump({"headline": result, "suite": rows}, f, indent=1)

    if not args.no_cpu_baseline:
        w16, x16 = WL.make_weight_and_x(m, batch)
        result["cpu_baseline"] = cpu_baseline(args, m, batch, w16, x16, nbytes)

    print(json.dumps(result), flush=True)


def kernel_label(m, batch):
    """Name of the kernel the library dispatches for this call (labels only)."""
    units = m.cols // 64
    if batch == 1:
        rpw = 2 if m.rows > 8192 else 1
        if units <= 256:
            return f"gemv_b1_direct_kernel<{m.n_keep},{rpw},{(units + 63) // 64},8>"
        return f"gemv_b1_kernel<{m.n_keep},{rpw},8>"
    if batch == 2 and m.rows <= 8192 and units <= 128:
        return f"gemv_bv_direct_kernel<{m.n_keep},2,{(units + 63) // 64}>"
    long_split = units > 256 and batch > 8 and m.rows <= 4096
    if units <= 512 and not (m.n_keep == 2 and long_split):
        return f"gemv_smfmac_rows_kernel<{m.n_keep},...>"
    if m.n_keep == 2:
        return "gemv_smfmac_split_kernel + gemv_split_reduce_kernel"
    return f"gemv_kernel<{m.n_keep},BT>=" + str(batch)


def run_suite(R, args):
    import workloads as WL
    out = []
    names = ("c1_512", "c2_4096", "c3_mlp7b", "c5_verify13b", "c4_stack7b", "x1_4096_1to4", "x2_mix_stack7b")
    stacks = ("c4_stack7b", "x2_mix_stack7b")
    if args.only:
        names = tuple(n for n in names if n in args.only.split(","))
    for name in names:
        wl = WL.WORKLOADS[name]
        mats = wl.matrices
        if name in stacks:
            # one outer and one inner layer individually; the whole stack below
            mats = [m for m in mats if m.name.startswith(("L0.", "L4."))]
        for m in mats:
            for b in wl.batches:
                r = R.measure_layer(m, b, args.suite_steps, max(1, args.suite_steps // 10), 3)
                r["workload"] = name
                print(f"suite {name}/{m.name} b{b}: cold {r['cold_us']:.2f} us ({r['cold_gbs']:.0f} GB/s), "
                      f"hot {r['hot_us']:.2f} us", file=sys.stderr, flush=True)
                out.append(r)
    for name in stacks:
        if args.no_stack or name not in names:
            continue
        for fused in (False, True):
            s = R.measure_stack(3, name, fused)
            s["workload"] = name + ("/all-fused" if fused else "/all")
            print(f"suite {s['workload']}: {s['us_per_pass']:.1f} us per {s['calls']}-call pass "
                  f"({s['gbs']:.0f} GB/s)", file=sys.stderr, flush=True)
            out.append(s)
    return out


def cpu_baseline(args, m, batch, w16, x16, packed_bytes):
    """The oracle as it stands, on this host's cores, on a bounded sample."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    ref = O.pack(w16, m.n_keep, m.group_size)
    t = time.perf_counter()
    w_hat = O.reconstruct(ref)
    recon_s = time.perf_counter() - t
    O.gemv(w_hat, x16)
    n = 0
    t = time.perf_counter()
    while True:
        O.gemv(w_hat, x16)
        n += 1
        el = time.perf_counter() - t
        if el >= args.cpu_seconds and n >= 3:
            break
    us = el / n * 1e6
    return {"value": round(packed_bytes / (us * 1e-6) / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "us_per_call": round(us, 1),
            "sample": f"{n} oracle GEMV calls (float64 W_hat @ x over the reconstructed {m.rows}x{m.cols} "
                      f"layer, plus the |W_hat|@|x| tolerance sums) in {el:.1f} s; reconstruction "
                      f"{recon_s:.2f} s once, not per call"}


if __name__ == "__main__":
    main()
