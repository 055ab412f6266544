#!/usr/bin/env python3
"""Benchmark libgemv on one MI355X.

One step is one GEMV call (the whole hot path: stage x, stream A once,
multiply-accumulate in fp32, reduce, add bias, write y) on the workload named
by ``--workload``; the default is the bf16 4096×4096 GEMV (the q/o
projection of the decode-layer sweep).  Inputs are seeded synthetic data
(no dataset or weights) and are resident in HBM before timing starts.

Cache defeat: ``R`` copies of A (and x, y) are allocated so that together
they exceed twice the 256 MB Infinity Cache, and consecutive steps cycle
through them, so every step streams its A from HBM.

Timed region: exactly ``--steps`` calls through the C ABI, bracketed by
``torch.cuda.synchronize()`` and a pair of HIP events on the launch stream.
The calls are enqueued while untimed lead-in work (replays of a HIP graph of
the same calls) keeps the GPU busy, after a warm-up of at least ``--warmup``
launches and 0.25 s, so they run back to back with no host gap between them
(host launch cost would otherwise exceed the ~5 µs kernel) and no graph
replay cost (about 10 µs per replay on this runtime).  ``value`` is
algorithmic bytes × steps ÷ elapsed; ``roofline.achieved`` divides the same
bytes by the average launch duration over that region; rocprofv3's kernel
trace of the same command gives the per-dispatch durations.  Also
measured:
  * eager calls through the C ABI (one ctypes call per step);
  * µs/call, GB/s and GFLOP/s for every other configured shape, including
    the fused decode calls (q/k/v as one multi-GEMV launch, gate/up with the
    SiLU product as one launch) and a whole decode layer's projections in
    four launches;
  * the CPU oracle on the host cores (``cpu_baseline``).

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
INFINITY_CACHE_BYTES = 256 << 20
METRIC = "achieved HBM GB/s (% of 8 TB/s) for 4096x4096 bf16 GEMV; µs/call per shape"
DEFAULT_WORKLOAD = "sweep_q"
SHAPE_WARMUP = 1000                # launches before each per-shape timed loop
# Before the timed region, graph replays run untimed for at least this long,
# whatever --warmup says (--warmup launches are a lower bound): a run of 20
# steps right after start-up read ~5 % slower than the same loop once the
# GPU had been busy for a while.
WARM_SECONDS = 0.25
LEAD_LAUNCHES = 256              # untimed launches in flight when timing starts


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--shapes", default="all",
                    help="comma-separated workloads for the per-shape table, 'all' or 'none'")
    ap.add_argument("--shape-steps", type=int, default=2000)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the CPU oracle timing (0 = skip)")
    ap.add_argument("--kernel-only", action="store_true",
                    help="only run the timed region of --workload, then as many launches "
                         "as event-timed graph replays (for profilers)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="CPU only: read the counter CSVs of the two --counters runs and write "
                         "the traffic summary used for roofline.traffic")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="time the read probe's variants (loads per lane, wavefronts per "
                         "workgroup, blocks per wavefront, cached/nontemporal, priority) over "
                         "rotated buffers of 8, 32 and 112 MiB, and the per-wavefront finish "
                         "times of the GEMV's own pattern; prints one JSON object")
    ap.add_argument("--shard-sweep", action="store_true",
                    help="time one GPU's share of the decode layer's seven projections when "
                         "2, 4 or 8 GPUs share it, cut by rows and by K (one GPU; collectives "
                         "not included); prints one JSON object")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="CPU only: per-kernel duration statistics of a rocprofv3 --kernel-trace "
                         "output directory (all dispatches, and the last --steps of each kernel: "
                         "the final graph replays of a --kernel-only run); prints one JSON object")
    ap.add_argument("--counters", action="store_true",
                    help="for rocprofv3 --pmc runs: a few eager launches of --workload over the "
                         "rotated buffers, then a plain device copy of COPY_BYTES for scaling")
    return ap.parse_args()


COPY_BYTES = 256 << 20   # the calibration copy: reads and writes this many bytes
PROFILES = os.path.join(ROOT, "profiles")


def source_code_only(text: str) -> str:
    """C++ source with its comments removed and whitespace runs collapsed
    (string and character literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":  # a literal: copy up to its closing quote
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of every HIP / host source of the library, comments and layout
    aside: counter figures taken from one version of the code are not
    reported for another."""
    import hashlib
    csrc = os.path.join(ROOT, "memory_bound_gemv_f32_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + source_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def summarize_counters(fetch_dir, write_dir, workload):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the GEMV kernel, scaled by
    the ratio of the calibration copy's known bytes to what the same counter
    read for it (the copy is the largest copy dispatch of the run)."""
    import csv
    out = {"workload": workload, "source_hash": kernel_source_hash(), "copy_bytes": COPY_BYTES}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))
        rows = [r for r in rows if r["Counter_Name"] == counter]
        gemv = [float(r["Counter_Value"]) for r in rows if "gemvdev::" in r["Kernel_Name"]]
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        scale = (COPY_BYTES / 1024) / copy
        key = counter.split("_")[0].lower()
        out[f"{key}_kib_per_dispatch"] = sum(gemv) / len(gemv)
        out[f"{key}_dispatches"] = len(gemv)
        out[f"copy_{key}_kib"] = copy
        out[f"{key}_scale"] = scale
        out[f"{key}_bytes_per_launch"] = sum(gemv) / len(gemv) * 1024 * scale
    out["traffic_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    return out


def summarize_trace(trace_dir, steps):
    """Duration statistics (ns) per kernel from rocprofv3's kernel trace:
    over every dispatch, and over each kernel's last `steps` dispatches (in
    a --kernel-only run, its final event-timed graph replays)."""
    import csv
    import numpy as np
    rows = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))))
    by = {}
    for r in rows:
        d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        by.setdefault(r["Kernel_Name"], []).append((int(r["Start_Timestamp"]), d))

    def stats(d):
        d = np.asarray(d, dtype=np.float64)
        return {"calls": int(d.size), "mean": round(float(d.mean()), 1),
                "p10": round(float(np.percentile(d, 10)), 1),
                "p50": round(float(np.percentile(d, 50)), 1),
                "p90": round(float(np.percentile(d, 90)), 1),
                "min": round(float(d.min()), 1), "max": round(float(d.max()), 1)}
    out = {}
    for name, v in by.items():
        v.sort()
        d = [x[1] for x in v]
        out[name] = {"all": stats(d), "last": stats(d[-steps:])}
    return out


def load_traffic(workload: str):
    """The stored counter traffic for this workload, or None if there is none
    or it was measured on other kernel sources."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t


def counters_run(case, rot, lg, torch):
    """Eager launches (one dispatch each) for per-dispatch counters, then a
    plain copy kernel of known size whose counter readings give the scale."""
    fns = rot.callers(lg, torch.cuda.current_stream().cuda_stream)
    for i in range(2 * rot.R):
        call(fns[i % len(fns)])
    torch.cuda.synchronize()
    n = COPY_BYTES // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    # evict src from the caches with an unrelated fill of > 2x the Infinity Cache
    junk = torch.empty(3 * INFINITY_CACHE_BYTES // 4, dtype=torch.float32, device="cuda").fill_(2.0)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del junk
    log(f"counters: {2 * rot.R} launches of the workload, then one {COPY_BYTES} B device copy")


class Rotation:
    """R device copies of one case's inputs/outputs, R chosen so that the
    copies of A together exceed 2× the Infinity Cache."""

    def __init__(self, case, torch, min_bytes=2 * INFINITY_CACHE_BYTES, splitk=False):
        import numpy as np
        self.case = case
        self.splitk = splitk  # run through gemv_splitk_* (one shared workspace)
        a_bytes = case.A.nbytes
        self.R = max(2, math.ceil(min_bytes / max(a_bytes, 1)) + 1)
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[case.dtype]
        if case.dtype == "f32":
            hA = torch.from_numpy(case.A.astype(np.float32))
            hX = torch.from_numpy(case.X.astype(np.float32))
        else:
            hA = torch.from_numpy(case.A.view(np.int16)).view(tdt)
            hX = torch.from_numpy(case.X.view(np.int16)).view(tdt)
        self.A, self.X, self.Y = [], [], []
        for _ in range(self.R):
            self.A.append(hA.to("cuda"))
            self.X.append(hX.to("cuda"))
            self.Y.append(torch.empty((case.nvec, case.M), dtype=torch.float32, device="cuda"))
        self.bias = None
        if case.bias is not None:
            self.bias = torch.from_numpy(case.bias).to("cuda")
        self.bytes_resident = self.R * (a_bytes + case.X.nbytes + 4 * case.M * case.nvec)
        self.ws = None
        if splitk:
            import memory_bound_gemv_f32_amd as lg
            n = lg.splitk_workspace_size(case.dtype, case.M, case.K)
            self.ws = torch.empty(max(n // 4, 1), dtype=torch.float32, device="cuda")

    def callers(self, lg, stream_handle):
        """One zero-argument callable per set that enqueues one call through
        the C ABI (arguments pre-marshalled, so a call is one ctypes call)."""
        c = self.case
        fns = []
        bias = self.bias.data_ptr() if self.bias is not None else None
        for i in range(self.R):
            A, X, Y = self.A[i].data_ptr(), self.X[i].data_ptr(), self.Y[i].data_ptr()
            if self.splitk:
                f = {"f32": lg.gemv_splitk_f32, "f16": lg.gemv_splitk_f16,
                     "bf16": lg.gemv_splitk_bf16}[c.dtype]
                ws = self.ws
                args = (A, c.lda, X, bias, Y, c.M, c.K, 0, ws.data_ptr(),
                        ws.numel() * 4, stream_handle)
            elif c.nvec > 1:
                f = {"f16": lg.gemv_batched_f16, "bf16": lg.gemv_batched_bf16}[c.dtype]
                args = (A, c.lda, X, bias, Y, c.M, c.K, c.nvec, stream_handle)
            else:
                f = {"f32": lg.gemv_f32, "f16": lg.gemv_f16, "bf16": lg.gemv_bf16}[c.dtype]
                args = (A, c.lda, X, bias, Y, c.M, c.K, stream_handle)
            fns.append((f, args))
        return fns


FUSED = ("fused_qkv", "fused_gate_up")


def fused_bytes(kind, parts, gi):
    """Algorithmic bytes of a fused call: every matrix once, x once, the
    outputs once in fp32 (q/k/v: one output per matrix; gate/up: h)."""
    n_out = sum(p.M for p in parts) if kind == "fused_qkv" else parts[0].M
    return (sum(p.M * p.K * gi.ELEMENT_BYTES[p.dtype] for p in parts) +
            parts[0].K * gi.ELEMENT_BYTES[parts[0].dtype] + 4 * n_out)


class FusedRotation:
    """R device sets of a fused decode problem: q/k/v as one multi-GEMV
    (``fused_qkv``) or the gate/up pair with the SiLU product
    (``fused_gate_up``); the matrices of one set share one x."""

    def __init__(self, kind, gi, torch, min_bytes=2 * INFINITY_CACHE_BYTES, parts=None):
        import numpy as np
        self.kind = kind
        if parts is None:
            parts = gi.make_fused_qkv() if kind == "fused_qkv" else list(gi.make_fused_gate_up())
        self.parts = parts
        p0 = self.parts[0]
        self.dtype, self.K = p0.dtype, p0.K
        a_bytes = sum(p.A.nbytes for p in self.parts)
        self.R = max(2, math.ceil(min_bytes / a_bytes) + 1)
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[p0.dtype]
        hA = [torch.from_numpy(p.A.view(np.int16)).view(tdt) for p in self.parts]
        hx = torch.from_numpy(p0.X[0].view(np.int16)).view(tdt)
        n_out = [p.M for p in self.parts] if kind == "fused_qkv" else [p0.M]
        self.sets = []
        for _ in range(self.R):
            self.sets.append(([a.to("cuda") for a in hA], hx.to("cuda"),
                              [torch.empty(m, dtype=torch.float32, device="cuda") for m in n_out]))
        self.bytes = fused_bytes(kind, self.parts, gi)
        self.M = sum(p.M for p in self.parts)

    def callers(self, lg, stream_handle):
        fns = []
        for As, x, ys in self.sets:
            if self.kind == "fused_qkv":
                table = lg.segment_table([(a.data_ptr(), p.lda, p.M, None, y.data_ptr())
                                          for a, p, y in zip(As, self.parts, ys)])
                f = {"f16": lg.gemv_multi_f16, "bf16": lg.gemv_multi_bf16}[self.dtype]
                args = (table, len(self.parts), x.data_ptr(), self.K, stream_handle)
            else:
                g, u = self.parts
                f = {"f16": lg.gemv_gate_up_silu_f16, "bf16": lg.gemv_gate_up_silu_bf16}[self.dtype]
                args = (As[0].data_ptr(), As[1].data_ptr(), g.lda, x.data_ptr(), ys[0].data_ptr(),
                        g.M, g.K, stream_handle)
            fns.append((f, args))
        return fns

    def sanity_check(self, torch):
        """Set 0 against torch's fp64 products on the device (the GEMV bound
        per row; for h the bound carried through silu and the product)."""
        As, x, ys = self.sets[0]
        xd = x.double()
        refs, sums = [], []
        for a, p in zip(As, self.parts):
            A = a.view(p.M, p.lda)[:, :p.K].double()
            refs.append(A @ xd)
            sums.append(A.abs() @ xd.abs())
        if self.kind == "fused_qkv":
            errs = [((y.double() - r).abs() / (1e-5 * sm + 1e-6)) for y, r, sm in zip(ys, refs, sums)]
            worst = max(float(e.max()) for e in errs)
        else:
            g, u = refs
            tg, tu = 1e-5 * sums[0] + 1e-6, 1e-5 * sums[1] + 1e-6
            sg = g * torch.sigmoid(g)
            h = sg * u
            bound = 1.1 * tg * (u.abs() + tu) + sg.abs() * tu + 1e-6 * h.abs() + 1e-6
            worst = float(((ys[0].double() - h).abs() / bound).max())
        return worst <= 1.0, worst


class Q8Rotation:
    """R device sets of a weight-only int8 problem (int8 Q, fp32 scales, x of
    a float type): y = scale ⊙ (Q·x) through gemv_q8_*."""

    def __init__(self, name, gi, torch, min_bytes=2 * INFINITY_CACHE_BYTES):
        import numpy as np
        self.case = c = gi.make_q8_workload(name)
        self.R = max(2, math.ceil(min_bytes / c.Q.nbytes) + 1)
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[c.xdtype]
        hQ = torch.from_numpy(np.ascontiguousarray(c.Q))
        hx = (torch.from_numpy(c.X[0].astype(np.float32)) if c.xdtype == "f32"
              else torch.from_numpy(c.X[0].view(np.int16)).view(tdt))
        self.scale = torch.from_numpy(c.scale).to("cuda")
        self.sets = [(hQ.to("cuda"), hx.to("cuda"),
                      torch.empty(c.M, dtype=torch.float32, device="cuda")) for _ in range(self.R)]

    def callers(self, lg, stream_handle):
        c = self.case
        f = {"f32": lg.gemv_q8_f32, "f16": lg.gemv_q8_f16, "bf16": lg.gemv_q8_bf16}[c.xdtype]
        return [(f, (Q.data_ptr(), c.ldq, self.scale.data_ptr(), x.data_ptr(), None,
                     y.data_ptr(), c.M, c.K, stream_handle)) for Q, x, y in self.sets]

    def sanity_check(self, torch):
        """Set 0 against torch's fp64 product on the device, within
        1e-5·|scale|·Σ|q·x| + 1e-6 per row."""
        c = self.case
        Q, x, y = self.sets[0]
        Qd = Q.view(c.M, c.ldq)[:, :c.K].double()
        xd = x.double()
        s = self.scale.double()
        ref = s * (Qd @ xd)
        bound = 1e-5 * s.abs() * (Qd.abs() @ xd.abs()) + 1e-6
        worst = float(((y.double() - ref).abs() / bound).max())
        return worst <= 1.0, worst


HOT_MAX_BYTES = 4 << 20   # shapes this small also get a cache-hot figure


class HotRotation:
    """Set 0 of a Rotation on every call: inputs stay in the caches."""

    def __init__(self, rot):
        self.rot = rot
        self.R = 1

    def callers(self, lg, stream_handle):
        return self.rot.callers(lg, stream_handle)[:1]


class ProbeRotation:
    """The read probe over the A buffers of a Rotation: every step streams
    one copy of A (no x, no output) with the GEMV kernels' access pattern."""

    def __init__(self, rot, torch):
        self.rot = rot
        self.R = rot.R
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def callers(self, lg, stream_handle):
        nbytes = self.rot.case.A.nbytes
        return [(lg.gemv_read_probe, (A.data_ptr(), nbytes, self.sink.data_ptr(), stream_handle))
                for A in self.rot.A]


class ProbeVariantRotation:
    """R buffers of `nbytes` (together more than 2x the Infinity Cache),
    each step streamed by one read-probe variant."""

    def __init__(self, torch, nbytes, min_bytes=2 * INFINITY_CACHE_BYTES):
        self.nbytes = nbytes
        self.R = max(2, math.ceil(min_bytes / nbytes) + 1)
        self.bufs = [torch.full((nbytes // 4,), 1, dtype=torch.int32, device="cuda")
                     for _ in range(self.R)]
        self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.variant = (8, 4, 1, 0)

    def callers(self, lg, stream_handle):
        loads, waves, blocks, flags = self.variant
        return [(lg.gemv_read_probe_variant, (b.data_ptr(), self.nbytes, self.sink.data_ptr(), loads,
                                              waves, blocks, flags, None, 0, stream_handle))
                for b in self.bufs]


PROBE_SIZES = {"8MiB": 8 << 20, "32MiB": 32 << 20, "112MiB": 112 << 20}
PROBE_ROUNDS = 5


def probe_variants():
    """(loads per lane, wavefronts per workgroup, blocks per wavefront, flags):
    flags bit 0 cached loads, bit 1 raised priority, bit 2 grid-stride."""
    out = [(8, 4, 1, 0)]  # the GEMV families' pattern (gemv_read_probe)
    for loads in (2, 4, 8, 16):
        for waves in (1, 2, 4, 8, 16):
            if (loads, waves) != (8, 4):
                out.append((loads, waves, 1, 0))
    for loads, waves in ((4, 4), (8, 4), (8, 8), (16, 4)):
        for blocks in (2, 4, 8):
            out.append((loads, waves, blocks, 4))
            out.append((loads, waves, blocks, 0))
    for v in ((8, 4, 1, 1), (8, 4, 1, 2), (8, 4, 1, 3), (4, 4, 1, 2), (16, 4, 1, 2), (8, 8, 1, 2),
              (8, 4, 2, 6), (8, 4, 4, 6)):
        out.append(v)
    return out


def probe_sweep(torch, lg, steps):
    """µs per launch of every read-probe variant at each size, graph loops of
    `steps` launches over rotated buffers; and, for the GEMV pattern, the
    spread of wavefront finish times within one launch."""
    import numpy as np
    result = {"steps": steps, "rounds": PROBE_ROUNDS, "sizes": {}, "wave_finish": {}}
    for label, nbytes in PROBE_SIZES.items():
        rot = ProbeVariantRotation(torch, nbytes)
        variants = probe_variants()
        times = {v: [] for v in variants}
        # rounds over all variants, so that drifts of the GPU's state spread
        # over every variant alike; the median of the rounds is reported
        for rnd in range(PROBE_ROUNDS):
            for v in variants:
                rot.variant = v
                loop = GraphLoop(torch, rot, lg, steps, per=rot.R * max(1, 256 // rot.R))
                times[v].append(1e3 * loop.time(warmup=min(steps, 500)) / steps)
                del loop
            log(f"probe {label}: round {rnd + 1} of {PROBE_ROUNDS} done")
        rows = []
        for v in variants:
            us = statistics.median(times[v])
            rows.append({"loads_per_lane": v[0], "waves_per_group": v[1], "blocks_per_wave": v[2],
                         "cached": bool(v[3] & 1), "priority": bool(v[3] & 2),
                         "grid_stride": bool(v[3] & 4), "us": round(us, 3),
                         "us_rounds": [round(t, 3) for t in times[v]],
                         "GBps": round(nbytes / us / 1e3, 1)})
            log(f"probe {label} {v}: {us:.3f} us, {nbytes / us / 1e3:.1f} GB/s")
        result["sizes"][label] = {"bytes": nbytes, "rotation_sets": rot.R, "variants": rows}
        # wavefront finish times of the GEMV pattern: one launch, timed per wavefront
        n_waves = -(-nbytes // (8 * 1024))
        times = torch.zeros(2 * n_waves + 64, dtype=torch.int64, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        for rep in range(3):
            b = rot.bufs[rep % rot.R]
            rc = lg.gemv_read_probe_variant(b.data_ptr(), nbytes, rot.sink.data_ptr(), 8, 4, 1, 0,
                                            times.data_ptr(), times.numel(), stream)
            if rc != 0:
                raise RuntimeError(f"gemv_read_probe_variant returned {rc}")
        torch.cuda.synchronize()
        t = times[:2 * n_waves].cpu().numpy().reshape(n_waves, 2).astype(np.int64)
        t0 = t[:, 0].min()
        start, end = (t[:, 0] - t0) * 10e-3, (t[:, 1] - t0) * 10e-3  # 100 MHz counter -> µs
        group = np.arange(n_waves) // 4
        xcd = group % 8
        late = end >= np.percentile(end, 90)
        result["wave_finish"][label] = {
            "waves": int(n_waves),
            "start_us_p50_p90_max": [round(float(np.percentile(start, q)), 3) for q in (50, 90, 100)],
            "end_us_p10_p50_p90_max": [round(float(np.percentile(end, q)), 3) for q in (10, 50, 90, 100)],
            "late_decile_share_by_xcd": [round(float((late & (xcd == i)).sum() / max(late.sum(), 1)), 3)
                                         for i in range(8)],
            "late_decile_mean_position": round(float(np.flatnonzero(late).mean() / n_waves), 3),
        }
        log(f"wave finish {label}: {result['wave_finish'][label]}")
        del rot, times
        torch.cuda.empty_cache()
    return result


SHARD_GPUS = (1, 2, 4, 8)


def fused_shard_layer(torch, lg, gi, G, steps):
    """One GPU's rows of the decode layer in four launches when G GPUs
    share it by rows: q/k/v in one multi-GEMV, o, gate/up with the SiLU
    product, down."""
    seeds = {n: 640 + i for i, n in enumerate(gi.SWEEP_SHAPES)}

    def part(name, x_of=None):
        M, K = gi.SWEEP_SHAPES[name]
        c = gi.make_random("bf16", M // G, K, seed=seeds[name], dist="normal", scale=0.02)
        if x_of is not None:
            c.X = x_of.X
        return c

    total_us, total_bytes, launches = 0.0, 0, {}
    q = part("q")
    gate = part("gate")
    for label, rot in (("qkv", lambda: FusedRotation("fused_qkv", gi, torch,
                                                     parts=[q, part("k", q), part("v", q)])),
                       ("o", lambda: Rotation(part("o"), torch)),
                       ("gate_up", lambda: FusedRotation("fused_gate_up", gi, torch,
                                                         parts=[gate, part("up", gate)])),
                       ("down", lambda: Rotation(part("down"), torch))):
        r = rot()
        call(r.callers(lg, torch.cuda.current_stream().cuda_stream)[0])
        torch.cuda.synchronize()
        if isinstance(r, FusedRotation):
            ok, worst = r.sanity_check(torch)
            nbytes = r.bytes
        else:
            ok, worst = sanity_check(r.case, r, torch)
            nbytes = r.case.algorithmic_bytes()
        if not ok:
            raise RuntimeError(f"fused layer shard {G} {label}: output check failed ({worst:.3g})")
        loop = GraphLoop(torch, r, lg, steps, per=r.R * max(1, 256 // r.R))
        us = 1e3 * loop.time(warmup=min(steps, 500)) / steps
        launches[label] = round(us, 3)
        total_us += us
        total_bytes += nbytes
        del loop, r
        torch.cuda.empty_cache()
    return {"us_per_gpu": round(total_us, 3), "GBps_per_gpu": round(total_bytes / total_us / 1e3, 1),
            "launches_us": launches}


def shard_sweep(torch, lg, gi, steps):
    """One GPU's share of the decode layer's seven bf16 projections when G
    GPUs share it, at the share's real shape: cut by rows (M/G × K: each GPU
    writes its own slice of y, no collective in the GEMV) or by K (M × K/G:
    each GPU writes a partial y for a sum all-reduce of 4·M bytes, not
    included here).  Graph loops of `steps` launches over rotated inputs per
    shape; every output checked against torch's fp64 product first."""
    out = {"steps": steps, "what": "us per launch of one GPU's share; collectives not included",
           "cuts": []}
    base = None
    for G in SHARD_GPUS:
        for cut in (("rows",) if G == 1 else ("rows", "k")):
            shapes, total_us, total_bytes = {}, 0.0, 0
            for i, (name, (M, K)) in enumerate(gi.SWEEP_SHAPES.items()):
                m, k = (M // G, K) if cut == "rows" else (M, K // G)
                case = gi.make_random("bf16", m, k, seed=640 + i, dist="normal", scale=0.02)
                rot = Rotation(case, torch)
                call(rot.callers(lg, torch.cuda.current_stream().cuda_stream)[0])
                torch.cuda.synchronize()
                ok, worst = sanity_check(case, rot, torch)
                if not ok:
                    raise RuntimeError(f"shard {G} {cut} {name}: output check failed ({worst:.3g})")
                loop = GraphLoop(torch, rot, lg, steps, per=rot.R * max(1, 256 // rot.R))
                us = 1e3 * loop.time(warmup=min(steps, 500)) / steps
                nbytes = case.algorithmic_bytes()
                plan = lg.plan("bf16", m, k, A_addr=rot.A[0].data_ptr(), X_addr=rot.X[0].data_ptr())
                shapes[name] = {"M": m, "K": k, "us": round(us, 3),
                                "GBps": round(nbytes / us / 1e3, 1),
                                "family": lg.FAMILY_NAMES.get(plan["family"], "?")}
                total_us += us
                total_bytes += nbytes
                del loop, rot
                torch.cuda.empty_cache()
            row = {"gpus": G, "cut": cut, "layer_us_per_gpu": round(total_us, 3),
                   "layer_GBps_per_gpu": round(total_bytes / total_us / 1e3, 1), "shapes": shapes}
            if cut == "rows":
                row["fused_layer"] = fused_shard_layer(torch, lg, gi, G, steps)
            if base is None:
                base = total_us
            row["speedup_vs_1_gpu"] = round(base / total_us, 3)
            row["efficiency"] = round(base / (G * total_us), 3)
            out["cuts"].append(row)
            log(f"shards: {G} GPUs by {cut}: {total_us:.3f} us per GPU for the layer "
                f"({row['speedup_vs_1_gpu']}x one GPU)"
                + (f"; in four fused launches {row['fused_layer']['us_per_gpu']:.3f} us"
                   if "fused_layer" in row else ""))
    return out


def call(fn_args):
    f, args = fn_args
    rc = f(*args)
    if rc != 0:
        raise RuntimeError(f"{f.__name__} returned {rc}")


def build_graph(torch, rot, lg, launches):
    """A HIP graph of ``launches`` back-to-back calls cycling through the
    rotation sets (captured from the C-ABI launches on a side stream)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fns = rot.callers(lg, s.cuda_stream)
        call(fns[0])  # warm the launch path outside capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(launches):
                call(fns[i % len(fns)])
    torch.cuda.synchronize()
    return g


class GraphLoop:
    """Exactly ``steps`` launches as replays of a main graph (``per`` calls)
    plus one tail graph for the remainder."""

    def __init__(self, torch, rot, lg, steps, per):
        self.torch = torch
        self.per = min(per, steps)
        self.replays, rem = divmod(steps, self.per)
        self.main = build_graph(torch, rot, lg, self.per)
        self.tail = build_graph(torch, rot, lg, rem) if rem else None
        self.steps = steps

    def run(self):
        for _ in range(self.replays):
            self.main.replay()
        if self.tail is not None:
            self.tail.replay()

    def warm(self, warmup, seconds=0.0):
        """Untimed replays: at least `warmup` launches and `seconds` of
        wall time; returns the launches run."""
        torch = self.torch
        n = 0
        t_end = time.perf_counter() + seconds
        while True:
            for _ in range(max(1, math.ceil(warmup / self.per))):
                self.main.replay()
                n += self.per
            torch.cuda.synchronize()
            if time.perf_counter() >= t_end:
                return n
            warmup = max(warmup, 100 * self.per)

    def time(self, warmup, seconds=0.0):
        torch = self.torch
        self.warm_launches = self.warm(warmup, seconds)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        # untimed lead-in replays keep the GPU busy while the host submits the
        # start event and the timed graphs, so the timed launches run back to
        # back from the start event on (recorded on an idle GPU, the graphs'
        # submission latency would land inside a short timed region)
        for _ in range(max(1, math.ceil(LEAD_LAUNCHES / self.per))):
            self.main.replay()
        e0.record()
        self.run()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)


def time_queued(torch, loop, fns, steps, warmup, seconds):
    """Exactly `steps` launches through the C ABI (one ctypes call each),
    enqueued while untimed graph replays keep the GPU busy, bracketed by an
    event pair on the launch stream: the launches run back to back with no
    host gap and no graph-replay cost between them.  (A graph replay costs
    about 10 µs of its own on this runtime: a short timed region of one
    replayed graph read ~0.5 µs per launch slower.)  Returns (ms, lead
    launches, whether the queue stayed ahead of the GPU)."""
    loop.warm(warmup, seconds)
    # per-launch GPU time and host cost per call, to size the lead-in
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    loop.main.replay()
    e1.record()
    torch.cuda.synchronize()
    gpu_us = 1e3 * e0.elapsed_time(e1) / loop.per
    t0 = time.perf_counter()
    for i in range(64):
        call(fns[i % len(fns)])
    host_us = 1e6 * (time.perf_counter() - t0) / 64
    torch.cuda.synchronize()
    lead = max(LEAD_LAUNCHES, math.ceil(4 * steps * host_us / max(gpu_us, 1e-3)))
    replays = math.ceil(lead / loop.per)
    ea = torch.cuda.Event(enable_timing=True)
    t_submit = time.perf_counter()
    ea.record()
    for _ in range(replays):
        loop.main.replay()
    e0.record()
    for i in range(steps):
        call(fns[i % len(fns)])
    t_submit = time.perf_counter() - t_submit
    e1.record()
    torch.cuda.synchronize()
    # the GPU started the lead-in about when the host started submitting it
    # (it was idle); the lead-in's GPU time must have outlasted the host's
    # submission of it and of the timed launches, or the GPU went idle
    # inside the timed region
    lead_ms = ea.elapsed_time(e0)
    return e0.elapsed_time(e1), replays * loop.per, 1e3 * t_submit < lead_ms


def time_eager(torch, fns, steps, warmup):
    for i in range(warmup):
        call(fns[i % len(fns)])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        call(fns[i % len(fns)])
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def sanity_check(case, rot, torch):
    """Set 0's output (every row) against torch's fp64 matrix product on the
    device, within 1e-5·Σ|a·x| + 1e-6 per row: a guard that
    the timed launches compute the right thing.  (Element-by-element parity
    with the oracle, at this size too, is what the GPU tests check.)"""
    A = rot.A[0].view(case.M, case.lda)[:, :case.K].double()
    X = rot.X[0].view(case.nvec, case.K).double()
    ref = X @ A.T.contiguous()
    absdot = X.abs() @ A.abs().T.contiguous()
    if rot.bias is not None:
        ref += rot.bias.double()
    err = (rot.Y[0].view(case.nvec, case.M).double() - ref).abs()
    bound = 1e-5 * absdot + 1e-6
    ok = bool(torch.all(err <= bound))
    worst = float((err / bound).max()) if err.numel() else 0.0
    return ok, worst


def rotation_for(name, gi, torch):
    """The rotation sets of any named shape: a plain, split-K, fused or
    int8 workload."""
    if name in FUSED:
        return FusedRotation(name, gi, torch)
    if name in gi.Q8_WORKLOADS:
        return Q8Rotation(name, gi, torch)
    return Rotation(gi.make_workload(name), torch, splitk=name in gi.SPLITK_WORKLOADS)


def measure_shape(name, torch, lg, gi, steps):
    fused = name in FUSED
    q8 = name in gi.Q8_WORKLOADS
    if fused:
        rot = FusedRotation(name, gi, torch)
        nbytes, dtype, M, K, nvec, has_bias = rot.bytes, rot.dtype, rot.M, rot.K, 1, False
    elif q8:
        rot = Q8Rotation(name, gi, torch)
        c = rot.case
        nbytes, dtype, M, K, nvec, has_bias = c.algorithmic_bytes(), f"int8 x {c.xdtype}", \
            c.M, c.K, 1, False
    else:
        case = gi.make_workload(name)
        rot = Rotation(case, torch, splitk=name in gi.SPLITK_WORKLOADS)
        nbytes, dtype, M, K = case.algorithmic_bytes(), case.dtype, case.M, case.K
        nvec, has_bias = case.nvec, case.bias is not None
    # loops of 400 launches read 1-5 % slower than loops of 2000 on the same
    # box (down projection 19.5-19.8 against 18.6 µs); shapes get the same
    # graph size, warm-up and step count as the headline workload
    loop = GraphLoop(torch, rot, lg, steps, per=rot.R * max(1, 256 // rot.R))
    ms, n = loop.time(warmup=SHAPE_WARMUP), steps
    fns = rot.callers(lg, torch.cuda.current_stream().cuda_stream)
    eager_ms = time_eager(torch, fns, steps, warmup=rot.R)
    if q8:
        call(fns[0])
        torch.cuda.synchronize()
        ok, worst = rot.sanity_check(torch)
        Q0, x0, _ = rot.sets[0]
        plan = lg.plan_q8(c.xdtype, M, K, c.ldq, Q0.data_ptr(), x0.data_ptr())
        family = lg.FAMILY_NAMES[plan["family"]] + " (int8 weights)"
    elif fused:
        call(fns[0])
        torch.cuda.synchronize()
        ok, worst = rot.sanity_check(torch)
        if name == "fused_qkv":  # the planner sees the concatenated rows
            p0 = rot.parts[0]
            plan = lg.plan(dtype, M, K, p0.lda, 1, rot.sets[0][0][0].data_ptr(),
                           rot.sets[0][1].data_ptr())
            family = lg.FAMILY_NAMES[plan["family"]] + " (multi)"
        else:
            family = "gated_silu"
    else:
        call(fns[0])
        torch.cuda.synchronize()
        ok, worst = sanity_check(case, rot, torch)
        if rot.splitk:
            plan = lg.plan_splitk(case.dtype, case.M, case.K, case.lda, 0,
                                  rot.A[0].data_ptr(), rot.X[0].data_ptr())
            family = f"{lg.FAMILY_NAMES[plan['family']]} ({plan['splits']} slices) + reduce"
        else:
            plan = lg.plan(case.dtype, case.M, case.K, case.lda, case.nvec,
                           rot.A[0].data_ptr(), rot.X[0].data_ptr())
            family = lg.FAMILY_NAMES[plan["family"]]
    hot_us = None
    if not fused and not q8 and not rot.splitk and case.algorithmic_bytes() <= HOT_MAX_BYTES:
        # the same buffers on every call (the caches stay warm), as the
        # SGEMV page's timing loop does
        hot = HotRotation(rot)
        hloop = GraphLoop(torch, hot, lg, steps, per=256)
        hot_us = round(1e3 * hloop.time(warmup=SHAPE_WARMUP) / steps, 3)
        del hloop, hot
    single_us = None
    if not fused and not q8 and rot.splitk:  # the same problem in one pass, for comparison
        rot.splitk = False
        single = GraphLoop(torch, rot, lg, steps, per=rot.R * max(1, 256 // rot.R))
        single_us = round(1e3 * single.time(warmup=SHAPE_WARMUP) / steps, 3)
        del single
    if not ok:
        raise RuntimeError(f"{name}: output outside the bound (worst error/bound {worst:.3g})")
    flops = gi.workload_flops(M, K, nvec, has_bias)
    us = 1e3 * ms / n
    del loop, rot
    torch.cuda.empty_cache()
    return {
        "dtype": dtype, "M": M, "K": K, "nvec": nvec,
        "bias": has_bias, "bytes": nbytes,
        "family": family,
        "us_per_call_graph": round(us, 3),
        "us_per_call_eager": round(1e3 * eager_ms / steps, 3),
        "GBps": round(nbytes / us / 1e3, 1),
        "frac_of_8TBps": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
        "GFLOPps": round(flops / us / 1e3, 1),
        **({"us_per_call_single_pass": single_us} if single_us is not None else {}),
        **({"us_per_call_graph_hot": hot_us,
            "GBps_hot": round(nbytes / hot_us / 1e3, 1)} if hot_us is not None else {}),
    }


def cpu_baseline(case, seconds):
    """The CPU oracle, as it stands, on the same workload: 1 warmup, then
    repeats until ``seconds`` of wall time; median."""
    import oracle
    o = oracle.default()
    o.gemv(case.dtype, case.A, case.X, case.bias, case.M, case.K, lda=case.lda, nvec=case.nvec)
    times = []
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or len(times) < 3:
        t0 = time.perf_counter()
        o.gemv(case.dtype, case.A, case.X, case.bias, case.M, case.K, lda=case.lda, nvec=case.nvec)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {
        "value": round(case.algorithmic_bytes() / med / 1e9, 3),
        "unit": "GB/s",
        "cores": o.num_threads(),
        "kind": "oracle",
        "sample": (f"the whole {case.dtype} {case.M}x{case.K} workload, {len(times)} repeats "
                   f"in {seconds:.0f} s after 1 warmup, median {med * 1e3:.2f} ms per call; "
                   "fp64 C loop, OpenMP over rows"),
    }


def main():
    args = parse()
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace, args.steps), indent=1))
        return
    if args.summarize_counters:
        t = summarize_counters(*args.summarize_counters, args.workload)
        os.makedirs(PROFILES, exist_ok=True)
        with open(traffic_file(args.workload), "w") as f:
            json.dump(t, f, indent=1)
            f.write("\n")
        print(json.dumps(t, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: every box in this setup has a single MI355X, "
              f"so --gpus {args.gpus} is not supported (the row-sharded multi-GPU layout is "
              f"described in the design notes).", file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import gemv_inputs as gi
    import memory_bound_gemv_f32_amd as lg

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    log(f"device {torch.cuda.get_device_name(0)} ({torch.cuda.get_device_properties(0).gcnArchName})")

    if args.probe_sweep:
        print(json.dumps(probe_sweep(torch, lg, args.steps)), flush=True)
        return

    if args.shard_sweep:
        print(json.dumps(shard_sweep(torch, lg, gi, args.steps)), flush=True)
        return

    if args.kernel_only:
        # only the timed region of one named shape (for profilers), timed as
        # the headline is: launches queued behind lead-in work after a warm-up
        krot = rotation_for(args.workload, gi, torch)
        kloop = GraphLoop(torch, krot, lg, args.steps, per=krot.R * max(1, 256 // krot.R))
        kfns = krot.callers(lg, torch.cuda.current_stream().cuda_stream)
        ms, lead, ahead = time_queued(torch, kloop, kfns, args.steps, args.warmup, WARM_SECONDS)
        log(f"kernel-only {args.workload}: {args.steps} launches, {1e3 * ms / args.steps:.3f} us "
            f"per launch (queue ahead of the GPU: {ahead})")
        # then the same number of launches as replayed graphs, event-timed: the
        # last `steps` dispatches of a trace of this run are these, back to
        # back on the GPU even under a tracer that slows the host
        gms = kloop.time(warmup=0)
        log(f"kernel-only {args.workload}: then {args.steps} launches as graph replays, "
            f"{1e3 * gms / args.steps:.3f} us per launch (event pair around the replays)")
        return

    case = gi.make_workload(args.workload)
    rot = Rotation(case, torch)
    log(f"workload {args.workload}: {case.dtype} M={case.M} K={case.K} nvec={case.nvec} "
        f"rotation sets {rot.R} ({rot.bytes_resident / 2**20:.0f} MiB resident)")
    loop = GraphLoop(torch, rot, lg, args.steps, per=rot.R * max(1, 256 // rot.R))
    if args.counters:
        counters_run(case, rot, lg, torch)
        return

    call(rot.callers(lg, torch.cuda.current_stream().cuda_stream)[0])
    torch.cuda.synchronize()
    ok, worst = sanity_check(case, rot, torch)
    log(f"check vs torch fp64 on the device (set 0, every row): {'ok' if ok else 'FAILED'}; "
        f"worst error / bound = {worst:.3g}")
    if not ok:
        sys.exit(1)

    # timed region: exactly --steps launches through the C ABI, queued behind
    # untimed lead-in work, after at least --warmup launches and WARM_SECONDS
    # of untimed replays
    fns = rot.callers(lg, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ms, lead_launches, queue_ahead = time_queued(torch, loop, fns, args.steps, args.warmup,
                                                 WARM_SECONDS)
    launches = args.steps
    nbytes = case.algorithmic_bytes()
    us_step = 1e3 * ms / launches
    value = nbytes / us_step / 1e3  # GB/s
    log(f"queued: {launches} launches in {ms:.3f} ms -> {us_step:.3f} us/step, {value:.1f} GB/s "
        f"(lead-in {lead_launches} launches; queue ahead of the GPU: {queue_ahead})")
    graph_ms = loop.time(args.warmup)
    log(f"graph replays: {1e3 * graph_ms / launches:.3f} us/step")

    eager_ms = time_eager(torch, fns, args.steps, args.warmup)
    log(f"eager: {1e3 * eager_ms / args.steps:.3f} us/step")
    # Average launch duration over the timed region, from the event pair on
    # the launch stream: graph replays leave no host gap between launches,
    # so this is the launches' own back-to-back duration (each includes the
    # runtime's fixed cost between dependent kernels); the committed
    # rocprofv3 kernel trace of the same command gives the per-dispatch
    # durations.  An event pair around a single launch would add the events'
    # own ~2 us.
    k_mean = us_step
    achieved = nbytes / k_mean / 1e3

    plan = lg.plan(case.dtype, case.M, case.K, case.lda, case.nvec,
                   rot.A[0].data_ptr(), rot.X[0].data_ptr())
    # the practical ceiling: the same A buffers streamed by the read probe,
    # timed the same way as the GEMV
    probe = ProbeRotation(rot, torch)
    ploop = GraphLoop(torch, probe, lg, args.steps, per=rot.R * max(1, 256 // rot.R))
    pfns = probe.callers(lg, torch.cuda.current_stream().cuda_stream)
    probe_ms, _, _ = time_queued(torch, ploop, pfns, args.steps, args.warmup, WARM_SECONDS)
    probe_us = 1e3 * probe_ms / args.steps
    a_bytes = case.A.nbytes
    read_probe = {
        "bytes": a_bytes, "us": round(probe_us, 3),
        "GBps": round(a_bytes / probe_us / 1e3, 1),
        "frac_of_8TBps": round(a_bytes / probe_us / 1e3 / HBM_PEAK_GBS, 4),
        "gemv_us_over_probe_us": round(us_step / probe_us, 3),
        "what": "gemv_read_probe over the same rotated A buffers: A streamed once with the "
                "GEMV access pattern, no x, no output",
    }
    log(f"read probe: {probe_us:.3f} us for the {a_bytes} A bytes; GEMV/probe time "
        f"{us_step / probe_us:.3f}")
    del loop, ploop, probe, rot
    torch.cuda.empty_cache()

    t = load_traffic(args.workload)
    if t is None:
        traffic_bytes = None
        traffic_note = "no counter figures for the current kernel sources"
    else:
        traffic_bytes = round(t["traffic_bytes_per_launch"])
        traffic_note = (f"HBM-side bytes per launch from rocprofv3 FETCH_SIZE x {t['fetch_scale']:.3f} "
                        f"+ WRITE_SIZE x {t['write_scale']:.3f} (scales from a {COPY_BYTES} B copy); "
                        f"{traffic_bytes / nbytes:.4f} x the algorithmic bytes")

    shapes = {}
    names = [] if args.shapes == "none" else (
        list(gi.WORKLOADS) + list(FUSED) + list(gi.Q8_WORKLOADS) if args.shapes == "all"
        else args.shapes.split(","))
    for name in names:
        shapes[name] = measure_shape(name, torch, lg, gi, args.shape_steps)
        log(f"  {name}: {shapes[name]}")
    sweep = [n for n in shapes if n.startswith("sweep_")]
    sweep_agg = None
    if len(sweep) == len(gi.SWEEP_SHAPES):
        tb = sum(shapes[n]["bytes"] for n in sweep)
        tus = sum(shapes[n]["us_per_call_graph"] for n in sweep)
        sweep_agg = {"bytes": tb, "us": round(tus, 3), "GBps": round(tb / tus / 1e3, 1),
                     "frac_of_8TBps": round(tb / tus / 1e3 / HBM_PEAK_GBS, 4)}

    # one decode layer's projections: q/k/v fused, o, gate/up fused with the
    # SiLU product, down; against the same matrices as seven plain GEMVs
    layer = None
    if all(n in shapes for n in ("fused_qkv", "sweep_o", "fused_gate_up", "sweep_down")):
        parts = ("fused_qkv", "sweep_o", "fused_gate_up", "sweep_down")
        tb = sum(shapes[n]["bytes"] for n in parts)
        tus = sum(shapes[n]["us_per_call_graph"] for n in parts)
        layer = {"launches": 4, "bytes": tb, "us": round(tus, 3), "GBps": round(tb / tus / 1e3, 1),
                 "frac_of_8TBps": round(tb / tus / 1e3 / HBM_PEAK_GBS, 4)}
        if sweep_agg is not None:
            layer["speedup_vs_7_plain_gemvs"] = round(sweep_agg["us"] / tus, 3)

    cpu = None
    if args.cpu_seconds > 0:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(case, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": launches,
        "warmup": args.warmup,
        "ms_per_step": round(ms / launches, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded, resident in HBM, rotated over >2x the Infinity Cache)",
        "config": {
            "workload": f"{case.dtype} GEMV y=A·x, A {case.M}x{case.K} row-major, fp32 "
                        f"accumulate and output, no bias ({args.workload})",
            "M": case.M, "K": case.K, "nvec": case.nvec,
            "family": lg.FAMILY_NAMES[plan["family"]],
            "timing": ("back-to-back launches through the C ABI, queued behind untimed lead-in "
                       "work (graph replays) after a warm-up of at least 0.25 s; event pair on "
                       "the launch stream"),
            "lead_in_launches": lead_launches,
            "queue_stayed_ahead": queue_ahead,
            "us_per_call": round(us_step, 3),
            "us_per_call_graph_replays": round(1e3 * graph_ms / launches, 3),
            "us_per_call_eager": round(1e3 * eager_ms / args.steps, 3),
            "frac_of_8TBps": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_bytes,
            "traffic_note": traffic_note,
            "us_per_launch_events": round(k_mean, 3),
            "us_per_launch_what": "mean over the timed region of back-to-back launches, HIP "
                                  "events on the launch stream",
            "bytes_per_launch": nbytes,
        },
        "cpu_baseline": cpu,
        "read_probe": read_probe,
        "per_shape": shapes,
        "sweep_aggregate": sweep_agg,
        "decode_layer_fused": layer,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
