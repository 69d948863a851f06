"""Benchmark of the packed INT4 2-bit-CSR SparseGEMV on one MI355X.

One step = one ``i4s_run_ws`` call (the whole per-call hot path: stage x, stream
the packed weights, decode, multiply-accumulate, reduce, store y) over one
batch of synthetic input.  The layer is packed once beforehand (packing is
offline work); its time is reported separately as ``pack_ms``.

Cold (the headline): the packed layer is copied P = ceil(1 GiB / packed
bytes) times (byte-identical device copies, > 4x the 256 MB last-level
cache) and the steps visit the copies round-robin; before every timed trial
an untimed 512 MiB read evicts the caches, so no copy is still cached when a
trial starts, whatever the step count.  Hot (reported, labelled
cache-resident): one copy, no eviction.

Timing: a trial enqueues, on one stream, (the eviction read), a bounded
delay kernel, event e0, exactly K calls, event e1.  The delay keeps the GPU
busy while the host enqueues the calls, so e0..e1 spans the K calls running
back to back, not the host's launch rate (``queued`` says whether the host
finished enqueueing before the delay ended).  Per call = (e1 - e0) / K; the
median over trials is reported, and ``value``, ``ms_per_step``,
``pct_of_peak`` and ``roofline`` all come from that one figure.  Wall time
around each trial (torch.cuda.synchronize() on both sides) is reported as
well.  (Replaying a captured HIP graph instead adds about 10 us per replay
on this system, 0.5 us per call at K = 20; the events bracketing eager
launches add about 3 us per trial.)

Prints ONE JSON line for the 4096x4096 2:4 G128 batch-1 layer.  ``value`` is
packed bytes per call / seconds per call (GB/s, decimal) in cold mode.
``--suite FILE`` additionally measures every workload (all matrices and
batch sizes, each batch-1 layer next to a read-only launch of its own bytes,
the 224-call 7B stacks per layer and per pass) and writes a table.
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
CSRC = os.path.join(ROOT, "int4_sparse_gemv_amd", "csrc")
# the batch-1 kernel's sources: a profile is used only while they are unchanged
B1_SRCS = [os.path.join(CSRC, f) for f in ("i4s_gemv_b1.hip", "i4s_gemv_common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_c2_4096.json")
KTIME_FILE = os.path.join(ROOT, "profiles", "kernel_time_gemv_c2_4096.json")
FLUSH_BYTES = 512 << 20  # > 2x the last-level cache
# read-only launch shapes tried for the floor: (16-byte loads per lane,
# threads per block, blocks; 0 = one block per slab of the data)
FLOOR_SHAPES = [(v, t, 0) for t in (256, 512, 1024) for v in (1, 2, 4, 8)] + \
               [(4, 512, 256), (4, 512, 512), (2, 1024, 256), (8, 256, 1024), (2, 512, 1024)]


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
    ap.add_argument("--suite", default=None, help="also measure every workload and write a table here")
    ap.add_argument("--no-stack", action="store_true", help="with --suite: skip the 224-matrix 7B stacks")
    ap.add_argument("--only", default=None, help="with --suite: comma-separated workloads to measure")
    ap.add_argument("--suite-steps", type=int, default=1000, help="with --suite: timed calls per layer and trial")
    ap.add_argument("--no-floors", action="store_true",
                    help="skip the read-only and latency floor measurements")
    ap.add_argument("--lib", default=None,
                    help="time this build of libi4s (e.g. one made with build --define ... --out PATH)")
    ap.add_argument("--batch-paths", action="store_true",
                    help="instead of the headline: 2:4 layers at batch 2, 3, 4 and 8, one JSON line")
    ap.add_argument("--stack", default=None,
                    help="instead of the headline: one 7B stack (c4_stack7b or x2_mix_stack7b), per pass and per layer")
    ap.add_argument("--summarize-rocprof", nargs=2, metavar=("DIR", "OUT"), default=None,
                    help="summarize rocprofv3 CSV output under DIR into the text file OUT (no GPU needed)")
    ap.add_argument("--min-calls", type=int, default=20, help="with --summarize-rocprof")
    return ap.parse_args()


def sha_of(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def say(msg):
    print(msg, file=sys.stderr, flush=True)


class Runner:
    """Packs layers and times queued sequences of i4s_run calls."""

    def __init__(self, args):
        import torch
        import int4_sparse_gemv_amd as I
        from int4_sparse_gemv_amd import _binding as B
        from int4_sparse_gemv_amd import build as BLD
        self.torch, self.I, self.B, self.args = torch, I, B, args
        # (the HIP runtime torch brings is loaded first, then the library)
        self.lib = B.load(os.path.abspath(args.lib)) if getattr(args, "lib", None) else B.load()
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.stream = torch.cuda.current_stream(self.dev)
        self.keep = []
        f = ctypes.CDLL(BLD.FLOOR_LIB)
        f.i4sf_stream_read.restype = ctypes.c_int
        f.i4sf_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p]
        f.i4sf_stream_read_shape.restype = ctypes.c_int
        f.i4sf_stream_read_shape.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        f.i4sf_chase.restype = ctypes.c_int
        f.i4sf_chase.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.c_void_p]
        f.i4sf_delay.restype = ctypes.c_int
        f.i4sf_delay.argtypes = [ctypes.c_uint32, ctypes.c_void_p]
        self.floor = f
        self.sink = torch.zeros(16, dtype=torch.int32, device=self.dev)
        self.flush_buf = torch.full((FLUSH_BYTES,), 0x5A, dtype=torch.uint8, device=self.dev)

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

    def evict(self):
        """One untimed read of FLUSH_BYTES: afterwards no earlier data is cached."""
        st = self.floor.i4sf_stream_read(self.flush_buf.data_ptr(), FLUSH_BYTES, 0, self.sink.data_ptr(),
                                         self.stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"i4sf_stream_read returned {st}")

    def launch(self, item, sh):
        """Enqueue one call: an i4s_run_ws argument tuple, or a callable
        taking the stream handle and returning a status."""
        st = item(sh) if callable(item) else self.lib.i4s_run_ws(*item, sh)
        if st != 0:
            raise self.B.I4SError(st, "i4s_run")

    def run_timed(self, seq, steps, evict):
        """One trial: (eviction), delay, e0, `steps` calls visiting seq
        round-robin, e1 -- all enqueued on the one stream before the delay
        ends.  Returns (device ms per step, wall ms per step, whether the host
        had enqueued everything before the delay ended)."""
        torch = self.torch
        sh = self.stream.cuda_stream
        delay_us = min(100000, 2000 + 20 * steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if evict:
            self.evict()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t1 = time.perf_counter()
        st = self.floor.i4sf_delay(delay_us, sh)
        if st != 0:
            raise RuntimeError(f"i4sf_delay returned {st}")
        e0.record(self.stream)
        n = len(seq)
        for i in range(steps):
            self.launch(seq[i % n], sh)
        e1.record(self.stream)
        submit_us = (time.perf_counter() - t1) * 1e6
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        return e0.elapsed_time(e1) / steps, wall / steps, submit_us < 0.8 * delay_us

    def timed(self, seq, steps, warmup, trials, evict):
        """Median over trials of the device time per call (ms) of `steps`
        calls visiting seq round-robin, after `warmup` untimed calls, plus the
        per-trial figures."""
        import numpy as np
        sh = self.stream.cuda_stream
        for i in range(warmup):
            self.launch(seq[i % len(seq)], sh)
        evs, walls, oks = [], [], []
        for _ in range(trials):
            ev, wall, ok = self.run_timed(seq, steps, evict)
            evs.append(ev)
            walls.append(wall)
            oks.append(ok)
        return {"ms": float(np.median(evs)), "wall_ms": float(np.median(walls)), "trials_ms": evs,
                "queued": all(oks)}

    def launch_floor_us(self, steps=2000, trials=3):
        """Per-launch time of a one-element fill kernel timed the same way (the dispatch floor)."""
        torch = self.torch
        t = torch.zeros(1, device=self.dev)

        def fill(sh):
            t.fill_(1.0)
            return 0
        return self.timed([fill], steps, 20, trials, False)["ms"] * 1e3

    def read_floor(self, nbytes, shapes, steps=2000, trials=3):
        """Cold and hot per-launch time (us) of read-only launches of nbytes
        for each shape (vpl, threads, blocks), timed like the GEMV."""
        torch = self.torch
        nb = nbytes // 16 * 16
        copies = max(4, math.ceil((1 << 30) / nb))
        bufs = [torch.full((nb,), 0x5A, dtype=torch.uint8, device=self.dev) for _ in range(copies)]
        out = []
        for vpl, threads, blocks in shapes:
            def item(i):
                buf = bufs[i % copies]
                return lambda sh, buf=buf: self.floor.i4sf_stream_read_shape(
                    buf.data_ptr(), nb, vpl, threads, blocks, self.sink.data_ptr(), sh)
            cold = self.timed([item(i) for i in range(copies)], steps, 20, trials, True)
            hot = self.timed([item(0)], steps, 20, trials, False)
            out.append({"vpl": vpl, "threads": threads, "blocks": blocks,
                        "cold_us": round(cold["ms"] * 1e3, 4), "hot_us": round(hot["ms"] * 1e3, 4)})
        del bufs
        torch.cuda.empty_cache()
        return out

    def latency_ns(self, trials=3):
        """One lane chasing 4000 dependent loads through a random cycle spread
        over 2 GiB (one entry per KiB)."""
        import numpy as np
        torch = self.torch
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
            st = self.floor.i4sf_chase(nxt.data_ptr(), nxt.numel(), hops, outv.data_ptr(), self.stream.cuda_stream)
            e1.record(self.stream)
            torch.cuda.synchronize()
            if st != 0:
                raise RuntimeError(f"i4sf_chase returned {st}")
            lat.append(e0.elapsed_time(e1) * 1e6 / hops)
        k0 = int((order == 0).nonzero()[0])
        expect = int(order[(k0 + hops) % M]) * spacing
        if int(outv.item()) != expect:
            raise RuntimeError(f"pointer chase ended at {int(outv.item())}, expected {expect}")
        del nxt, order
        torch.cuda.empty_cache()
        return float(np.median(lat))

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
        cold = self.timed(seq, steps, warmup, trials, True)
        hot = self.timed(seq[:1], steps, warmup, trials, False)
        del cps, seq
        self.keep.clear()
        torch.cuda.empty_cache()
        flops = 2 * (p.nnz) * batch
        cold_us, hot_us = cold["ms"] * 1e3, hot["ms"] * 1e3
        return {"matrix": m.name, "rows": m.rows, "cols": m.cols, "n_keep": m.n_keep, "group_size": p.group_size,
                "batch": batch, "packed_bytes": nbytes, "copies": n_cold, "pack_ms": round(pack_ms, 3),
                "cold_us": cold_us, "hot_us": hot_us, "cold_wall_us": cold["wall_ms"] * 1e3,
                "cold_trials_us": [round(t * 1e3, 4) for t in cold["trials_ms"]], "queued": cold["queued"],
                "cold_gbs": nbytes / (cold_us * 1e-6) / 1e9, "hot_gbs": nbytes / (hot_us * 1e-6) / 1e9,
                "cold_tflops": flops / (cold_us * 1e-6) / 1e12}

    def stack_items(self, name):
        import workloads as WL
        torch = self.torch
        items, total, groups = [], 0, {}
        for m in WL.WORKLOADS[name].matrices:
            w16, x16 = WL.make_weight_and_x(m, 1)
            p, _ = self.pack(w16, m)
            x = self.to_dev(x16)
            y = torch.empty(1, m.rows, dtype=torch.float16, device=self.dev)
            items.append((p, x, y, 1))
            total += p.packed_nbytes()
            groups[p.group_size] = groups.get(p.group_size, 0) + 1
        return items, total, groups

    def layer_calls(self, items, layer, fused):
        """The calls of one layer: 7 single calls, or (fused) q/k/v and
        gate/up as one i4s_run_multi call each (4 calls).  Fused projections
        read the same x, as in a model."""
        li = items[7 * layer: 7 * layer + 7]  # q, k, v, o, gate, up, down
        if not fused:
            return self.calls(li)
        seq = []
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
        return seq

    def measure_stack(self, trials, name="c4_stack7b", fused=False, items=None):
        """The 224 projections of a 32-layer 7B stack in layer order (2.7 GB
        per pass, so every call streams from HBM).  Per pass: the calls of a
        whole pass, timed like the GEMV.  Per layer: in one pass queued behind
        a delay kernel, an event after each layer's calls; a layer's time is
        the span between its two events (the events themselves add a little)."""
        import numpy as np
        torch = self.torch
        own = items is None
        if own:
            items, total, groups = self.stack_items(name)
        else:
            items, total, groups = items
        layers = len(items) // 7
        per_layer = [self.layer_calls(items, l, fused) for l in range(layers)]
        seq = [c for calls in per_layer for c in calls]
        r = self.timed(seq, len(seq), len(seq), trials, False)
        pass_us = r["ms"] * len(seq) * 1e3
        # per layer: one pass per trial, an event after each layer
        sh = self.stream.cuda_stream
        spans = []
        for _ in range(trials):
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(layers + 1)]
            st = self.floor.i4sf_delay(50000, sh)
            if st != 0:
                raise RuntimeError(f"i4sf_delay returned {st}")
            ev[0].record(self.stream)
            for l, calls in enumerate(per_layer):
                for item in calls:
                    self.launch(item, sh)
                ev[l + 1].record(self.stream)
            torch.cuda.synchronize()
            spans.append([ev[l].elapsed_time(ev[l + 1]) * 1e3 for l in range(layers)])
        layer_us = [float(v) for v in np.median(np.array(spans), axis=0)]
        layer_bytes = [sum(p.packed_nbytes() for p, _, _, _ in items[7 * l: 7 * l + 7]) for l in range(layers)]
        res = {"calls": len(seq), "fused": fused, "packed_bytes": total, "us_per_pass": pass_us,
               "us_per_layer": pass_us / layers, "gbs": total / (pass_us * 1e-6) / 1e9,
               "group_sizes": groups,
               "layers": [{"layer": l, "us": round(layer_us[l], 3), "bytes": layer_bytes[l],
                           "gbs": round(layer_bytes[l] / (layer_us[l] * 1e-6) / 1e9, 1)} for l in range(layers)],
               "per_layer_sum_us": round(sum(layer_us), 2)}
        del seq, per_layer
        self.keep.clear()
        if own:
            del items
            torch.cuda.empty_cache()
        return res


BATCH_PATH_LAYERS = (("c2_4096", "w"), ("c5_verify13b", "attn"), ("c5_verify13b", "up"))


def batch_paths(R, args):
    """Cold and hot us/call of 2:4 layers at batch 2, 3, 4 and 8 through the
    loaded build of the library, with the kernel each call ran."""
    import workloads as WL
    rows = []
    for wl, name in BATCH_PATH_LAYERS:
        m = next(mm for mm in WL.WORKLOADS[wl].matrices if mm.name == name)
        for b in (2, 3, 4, 8):
            r = R.measure_layer(m, b, args.steps, args.warmup, args.trials)
            say(f"{wl}/{name} {m.rows}x{m.cols} b{b}: cold {r['cold_us']:.3f} us, hot {r['hot_us']:.3f} us")
            rows.append({"layer": f"{m.rows}x{m.cols}", "batch": b, "cold_us": round(r["cold_us"], 4),
                         "hot_us": round(r["hot_us"], 4)})
    return {"lib": args.lib or "default", "steps": args.steps, "trials": args.trials, "rows": rows}


def summarize_rocprof(d, out, min_calls):
    """rocprofv3 CSV output (kernel traces, counter collections) -> a short text file.

    Kernel trace: runs of >= min_calls consecutive dispatches of one kernel
    and grid (median, mean and minimum duration), then per kernel over the
    whole run.  Counters: the mean per dispatch of every counter, per kernel
    and grid."""
    import csv
    import glob
    import statistics as st
    from collections import defaultdict
    lines = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*_kernel_trace.csv"), recursive=True)):
        rows = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Start_Timestamp"]))
        runs, cur, key = [], [], None
        for r in rows:
            k = (r["Kernel_Name"], r["Grid_Size_X"], r["Grid_Size_Y"], r["Workgroup_Size_X"])
            if k != key and cur:
                runs.append((key, cur))
                cur = []
            key = k
            cur.append(r)
        if cur:
            runs.append((key, cur))
        lines.append(f"# kernel trace {os.path.basename(f)}: runs of >= {min_calls} consecutive dispatches "
                     f"of one kernel and grid")
        lines.append("# n | median us | mean us | min us | grid x,y | block | kernel")
        for (name, gx, gy, wg), run in runs:
            if len(run) < min_calls:
                continue
            du = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in run]
            lines.append(f"{len(run)} | {st.median(du):.3f} | {st.mean(du):.3f} | {min(du):.3f} | {gx},{gy} | {wg} | "
                         f"{name[:160]}")
        agg = defaultdict(list)
        for r in rows:
            agg[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines.append("# per kernel over the whole run: calls | mean us | median us | kernel")
        for name, du in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"{len(du)} | {st.mean(du):.3f} | {st.median(du):.3f} | {name[:160]}")
    for f in sorted(glob.glob(os.path.join(d, "**", "*_counter_collection.csv"), recursive=True)):
        vals = defaultdict(lambda: defaultdict(list))
        disp = defaultdict(set)
        for r in csv.DictReader(open(f)):
            key = (r["Kernel_Name"], r.get("Grid_Size", r.get("Grid_Size_X", "")))
            vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
            disp[key].add(r["Dispatch_Id"])
        lines.append(f"# counters {os.path.basename(f)}: mean per dispatch, kernels with >= {min_calls} dispatches")
        for key, cv in sorted(vals.items(), key=lambda kv: kv[0][0]):
            if len(disp[key]) < min_calls:
                continue
            cs = ", ".join(f"{c}={st.mean(v):.6g}" for c, v in sorted(cv.items()))
            lines.append(f"{len(disp[key])} dispatches | grid {key[1]} | {key[0][:160]} | {cs}")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    if args.summarize_rocprof:
        summarize_rocprof(*args.summarize_rocprof, args.min_calls)
        return
    import workloads as WL

    R = Runner(args)
    if args.batch_paths:
        print(json.dumps(batch_paths(R, args)), flush=True)
        return
    if args.stack:
        items = R.stack_items(args.stack)
        out = {"workload": args.stack, "passes": [R.measure_stack(args.trials, args.stack, f, items=items)
                                                  for f in (False, True)]}
        print(json.dumps(out), flush=True)
        return
    wl = WL.WORKLOADS[args.workload]
    m = wl.matrices[0] if args.matrix is None else next(mm for mm in wl.matrices if mm.name == args.matrix)
    batch = args.batch or wl.batches[0]

    head = R.measure_layer(m, batch, args.steps, args.warmup, args.trials)
    say(f"headline: {head['cold_us']:.4f} us/call cold, {head['hot_us']:.4f} hot, queued {head['queued']}")
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
    us = head["cold_us"]
    achieved = nbytes / (us * 1e-6) / 1e9
    src_sha = sha_of(B1_SRCS)
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if (tr.get("kernel_source_sha") == src_sha and tr.get("workload") == args.workload
                and tr.get("batch") == batch):
            traffic = tr.get("hbm_bytes_per_launch")
    kernel_only = None
    if os.path.exists(KTIME_FILE):
        with open(KTIME_FILE) as f:
            kt = json.load(f)
        if (kt.get("kernel_source_sha") == src_sha and kt.get("workload") == args.workload
                and kt.get("batch") == batch):
            kernel_only = {k: kt[k] for k in ("kernel", "avg_us", "calls", "profile", "kernel_source_sha")
                           if k in kt}
    kname = kernel_label(m, batch)

    result = {
        "metric": METRIC,
        "value": round(achieved, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us * 1e-3, 7),
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
            "mode": "cold", "copies": head["copies"], "timing": "stream launches queued behind a delay kernel",
            "packed_bytes": nbytes, "x_bytes": 2 * batch * m.cols, "y_bytes": 2 * batch * m.rows,
        },
        "us_per_call": round(us, 4),
        "pct_of_peak": round(100 * achieved / PEAK_HBM_GBS, 2),
        "trials_us": head["cold_trials_us"],
        "queued": head["queued"],
        "wall_us_per_call": round(head["cold_wall_us"], 4),
        "hot": {"us_per_call": round(head["hot_us"], 4), "gbs": round(head["hot_gbs"], 2),
                "note": "one copy, cache-resident (L2/MALL), not an HBM figure"},
        "launch_floor_us": round(floor_us, 4),
        "pack_ms": head["pack_ms"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": kname,
                     "algorithmic_bytes_per_launch": nbytes},
        "kernel_only": kernel_only,
    }

    if not args.no_floors:
        shapes = R.read_floor(nbytes, FLOOR_SHAPES)
        best = min(shapes, key=lambda s: s["cold_us"])
        plain = R.read_floor(nbytes, [(1, 256, 0)], trials=3)[0]
        result["floors"] = {
            "bytes": nbytes // 16 * 16,
            "read_only_shapes": shapes,
            "best_shape": {k: best[k] for k in ("vpl", "threads", "blocks")},
            "read_only_cold_us": best["cold_us"],
            "read_only_hot_us": best["hot_us"],
            "one_load_per_lane_cold_us": plain["cold_us"],
            "read_only_ceiling_gbs": round(nbytes / (best["cold_us"] * 1e-6) / 1e9, 2),
            "gemv_frac_of_read_only_ceiling": round(best["cold_us"] / us, 4),
            "empty_launch_us": round(floor_us, 4),
            "load_latency_ns": round(R.latency_ns(), 2),
        }

    if args.suite:
        rows = run_suite(R, args, result.get("floors", {}).get("best_shape"))
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
    if batch == 2 and m.rows <= 8192 and units <= 64:
        return f"gemv_bv_direct_kernel<{m.n_keep},2,{(units + 63) // 64}>"
    if m.n_keep == 2 and _split_wanted(m.rows, units, batch):
        return "gemv_smfmac_slice_kernel + gemv_slice_reduce_kernel"
    if units <= 512:
        return f"gemv_smfmac_rows_kernel<{m.n_keep},...>"
    return f"gemv_kernel<{m.n_keep},BT>=" + str(batch)


def _split_wanted(rows, units, batch):
    """The library's rule for the 2:4 K split at batch >= 2 (i4s_plan.cpp,
    restated for the label; the workspace size the library reports is the
    authority)."""
    tiles = (rows + 15) // 16
    if units > 512:
        return True
    if 3 <= batch <= 8:
        rows_blocks = (tiles + 1) // 2 if tiles >= 300 else tiles
        return units >= 128 and (rows_blocks < 192 or (batch == 8 and rows_blocks <= 256))
    if batch > 8:
        return units >= 80 and tiles <= 512
    return False


def run_suite(R, args, floor_shape):
    import workloads as WL
    out = []
    names = ("c1_512", "c2_4096", "c3_mlp7b", "c5_verify13b", "c4_stack7b", "x1_4096_1to4", "x2_mix_stack7b")
    stacks = ("c4_stack7b", "x2_mix_stack7b")
    if args.only:
        names = tuple(n for n in names if n in args.only.split(","))
    shapes = [(1, 256, 0), (2, 512, 0), (4, 512, 0)]
    if floor_shape and tuple(floor_shape.values()) not in shapes:
        shapes.append((floor_shape["vpl"], floor_shape["threads"], floor_shape["blocks"]))
    for name in names:
        wl = WL.WORKLOADS[name]
        mats = wl.matrices
        if name in stacks:
            # one outer and one inner layer individually; the whole stack below
            mats = [m for m in mats if m.name.startswith(("L0.", "L4."))]
        for m in mats:
            floor = None
            for b in wl.batches:
                r = R.measure_layer(m, b, args.suite_steps, max(1, args.suite_steps // 10), 3)
                r["workload"] = name
                if floor is None:
                    fl = R.read_floor(r["packed_bytes"], shapes, steps=args.suite_steps)
                    floor = min(fl, key=lambda s: s["cold_us"])
                r["read_only_cold_us"] = floor["cold_us"]
                r["read_only_shape"] = [floor["vpl"], floor["threads"], floor["blocks"]]
                r["frac_of_read_only"] = round(floor["cold_us"] / r["cold_us"], 4)
                say(f"suite {name}/{m.name} b{b}: cold {r['cold_us']:.2f} us ({r['cold_gbs']:.0f} GB/s), "
                    f"hot {r['hot_us']:.2f} us, read-only {floor['cold_us']:.2f} us")
                out.append(r)
    for name in stacks:
        if args.no_stack or name not in names:
            continue
        items = R.stack_items(name)
        for fused in (False, True):
            s = R.measure_stack(3, name, fused, items=items)
            s["workload"] = name + ("/all-fused" if fused else "/all")
            say(f"suite {s['workload']}: {s['us_per_pass']:.1f} us per {s['calls']}-call pass "
                f"({s['gbs']:.0f} GB/s); per-layer sum {s['per_layer_sum_us']:.1f} us")
            out.append(s)
        del items
        R.torch.cuda.empty_cache()
    return out


def cpu_baseline(args, m, batch, w16, x16, packed_bytes):
    """The oracle as it stands, on this host's cores, on a bounded sample:
    its pack of the layer once, its reconstruction once, then 3 warm-up and
    at least 10 timed GEMV calls (until cpu_seconds have passed); the median
    call is reported."""
    import numpy as np
    import oracle as O
    blas, threads = "unknown", len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if info:
            threads = max(d.get("num_threads", 1) for d in info)
            blas = ", ".join(f"{d.get('internal_api')} {d.get('version')}" for d in info)
    except Exception:  # pragma: no cover
        pass
    t = time.perf_counter()
    ref = O.pack(w16, m.n_keep, m.group_size)
    pack_s = time.perf_counter() - t
    t = time.perf_counter()
    w_hat = O.reconstruct(ref)
    recon_s = time.perf_counter() - t
    for _ in range(3):
        O.gemv(w_hat, x16)
    reps = []
    t_all = time.perf_counter()
    while len(reps) < 10 or time.perf_counter() - t_all < args.cpu_seconds:
        t = time.perf_counter()
        O.gemv(w_hat, x16)
        reps.append(time.perf_counter() - t)
    us = float(np.median(reps)) * 1e6
    return {"value": round(packed_bytes / (us * 1e-6) / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "us_per_call": round(us, 1), "blas": blas,
            "oracle_pack_s": round(pack_s, 3), "reconstruct_s": round(recon_s, 3),
            "sample": f"median of {len(reps)} oracle GEMV calls after 3 warm-ups (float64 W_hat @ x over the "
                      f"reconstructed {m.rows}x{m.cols} layer, plus the |W_hat|@|x| tolerance sums), "
                      f"{sum(reps):.1f} s in all; the oracle's pack ({pack_s:.2f} s) and reconstruction "
                      f"({recon_s:.2f} s) once, not per call"}


if __name__ == "__main__":
    main()
