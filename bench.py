#!/usr/bin/env python3
"""Benchmark of the batch-1 ternary bit-plane GEMV on one MI355X.

One step = one decode step's ternary GEMVs: the 210 matrices of BitNet b1.58 2B4T (30 layers x
q, k, v, o, gate, up, down), each applied to its own int8 activation, as one grouped launch
(activation staging + the weight-streaming GEMV). Inputs are seeded synthetic data of the
model's shapes and zero density; they are resident in HBM before timing starts. The weight set
is held in several HBM copies used in rotation, so no step finds the previous step's weights in
the 256 MB last-level cache: every step streams its 521,011,200 plane bytes from HBM.

Prints one JSON line: weight GB/s over the timed steps (value), microseconds per step, the
dominant kernel's roofline (HIP events around each GEMV launch), the CPU oracle's rate on the
host cores, and the companion measurements of the same workload family: streaming-read probe,
bf16 dense head, zero-density sweep and small-batch GEMM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Ternary GEMV weight GB/s (% HBM peak) + µs/decode-step, 2B4T shapes"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
BASE_SEED = 0x2B47
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_bitserial_decode_step_traffic.json")
# sources of the decode-step GEMV kernel; the committed counter summary holds their hash
KERNEL_SRCS = [os.path.join(ROOT, "bit_plane_weight_amd", "csrc", f)
               for f in ("bpw_gemv.hip", "bpw_gemv_tile.h", "bpw_device.h", "bpw_internal.h")]
# the BITCOS GEMV kernel: its VALU instruction count per decode-step launch, from a committed counter
# run on the same sources
BITCOS_FILE = os.path.join(ROOT, "profiles", "gemv_bitcos_decode_step_counters.json")
BITCOS_SRCS = [os.path.join(ROOT, "bit_plane_weight_amd", "csrc", f)
               for f in ("bpw_bitcos.hip", "bpw_device.h", "bpw_internal.h")]
# Integer VALU issue peak of MI355X: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz (a wave64
# VALU instruction occupies its SIMD for 4 clocks), in lane-operations per second.
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
LEGS = ("configs", "prologue", "intmlp", "small_batch_decode_step", "bitcos", "probe", "head", "z_sweep", "small_batch")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(paths=None) -> str:
    """SHA-256 of the kernel's sources and of the compiler flags its translation unit (the first path)
    is built with, so a record taken from another build of the same sources does not match."""
    from bit_plane_weight_amd import build as bpw_build
    paths = paths or KERNEL_SRCS
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(bpw_build.flags_for(paths[0])).encode())
    return h.hexdigest()


def host_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


class DecodeSet:
    """The 210 matrices of one decode step in `copies` HBM copies, plus activations and outputs."""

    def __init__(self, bpw, torch, synth, dev, copies: int, p_zero: float, base: int, layers=None,
                 cpu_oracle=None):
        self.plane_bytes = 0
        self.weights = 0
        self.copies = []
        xs, outs, host_mats = [], [], []
        shapes = synth.decode_step_shapes()
        layer_cache = {}
        for (layer, proj, name, rows, cols) in shapes:
            src_layer = layer if layers is None else layers(layer)
            key = (src_layer, proj)
            case = layer_cache.get(key)
            if case is None:
                case = synth.ternary_case(base, src_layer, proj, rows, cols, p_zero)
                if layers is not None:
                    layer_cache[key] = case
            planes = bpw.bpw_pack_i8(case.w)
            if cpu_oracle is not None:
                cpu_oracle(case, layer)
            hm = bpw.bpw_load(planes, rows, cols, case.w_scale)
            host_mats.append(hm)
            x = torch.from_numpy(case.x).to(dev)  # cols is a multiple of 64: bpr * 64 bytes
            oi = torch.empty(rows, dtype=torch.int32, device=dev)
            of = torch.empty(rows, dtype=torch.float32, device=dev)
            xs.append((x, case.x_scale))
            outs.append((oi, of))
            self.plane_bytes += hm.nbytes
            self.weights += rows * cols
        for c in range(copies):
            mats = []
            for hm in host_mats:
                buf = torch.empty(hm.nbytes, dtype=torch.uint8, device=dev)
                mats.append(bpw.bpw_upload(hm, buf))
            jobs = [bpw.gemv_job(m, x, s, oi, of) for m, (x, s), (oi, of) in zip(mats, xs, outs)]
            ws = torch.empty(bpw.bpw_gemv_workspace_bytes(jobs), dtype=torch.uint8, device=dev)
            self.copies.append((bpw.GemvPlan(jobs, ws), mats, ws))
        self.shapes = shapes
        self.host_mats = host_mats  # freed by free_host()
        self.xs, self.outs = xs, outs

    def free_host(self):
        for hm in self.host_mats:
            hm.free()
        self.host_mats = []

    def plan(self, i):
        return self.copies[i % len(self.copies)][0]


def settle(torch, fn, min_ms: float = 40.0) -> None:
    """Run fn (a few launches) until min_ms of wall time has passed. Under sustained load the GPU's
    clocks take about 20 ms to ramp up (measured: 50-step blocks of the decode step at 103, 90, 84,
    82 us, then 81.5 us; again after 2 s idle), so every measurement that follows host work or idle
    time runs this first."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        torch.cuda.synchronize()


def time_steps(torch, dset, steps: int) -> tuple[float, float]:
    """Run `steps` decode steps back to back (one GEMV launch each, plans in rotation) between two
    HIP events on the launch stream. Returns (GPU ms per step from the events, wall ms per step);
    the GPU figure is the kernel's average duration plus the gap between consecutive launches."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record()
    for i in range(steps):
        dset.plan(i).run()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return a.elapsed_time(b) / steps, wall * 1e3 / steps


def prologue_measure(bpw, torch, synth, dev, ds, steps: int = 100) -> dict:
    """The decode step with its activation prep: the Folded quantiser turns each job's float32
    residual h and gain g (seeded: h ~ N(0, 1), g ~ U(0.5, 1.5)) into the job's int8 codes and a
    device-resident scale, then the grouped GEMV reads both. One quantiser launch (210 jobs) plus one
    GEMV launch per step, timed back to back between HIP events. Beside it, the plain streaming read of
    the quantiser's input bytes, timed the same way."""
    import numpy as np
    qjobs, scales, keep = [], [], []
    for i, ((layer, proj, name, rows, cols), (x, _)) in enumerate(zip(ds.shapes, ds.xs)):
        h = torch.from_numpy(synth.normal_f32(BASE_SEED + 31 * i + 1, cols)).to(dev)
        g = torch.from_numpy((np.float32(0.5) + synth.uniform(BASE_SEED + 31 * i + 2, cols)).astype(np.float32)).to(dev)
        sd = torch.zeros(1, dtype=torch.float32, device=dev)
        qjobs.append(bpw.quant_job(h, g, x, sd, 1e-5))
        scales.append(sd)
        keep += [h, g]
    qws = torch.empty(bpw.bpw_quantize_workspace_bytes(len(qjobs)), dtype=torch.uint8, device=dev)
    qplan = bpw.QuantPlan(qjobs, qws)
    plans = []
    for plan, mats, _ in ds.copies:
        jobs = [bpw.gemv_job(m, x, 0.0, oi, of, x_scale_dev=sd)
                for m, (x, _), (oi, of), sd in zip(mats, ds.xs, ds.outs, scales)]
        ws = torch.empty(bpw.bpw_gemv_workspace_bytes(jobs), dtype=torch.uint8, device=dev)
        plans.append((bpw.GemvPlan(jobs, ws), ws))
    def some():
        for i in range(10):
            qplan.run()
            plans[i % len(plans)][0].run()
    settle(torch, some)
    a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    a.record()
    for i in range(steps):
        qplan.run()
    b.record()
    for i in range(steps):
        qplan.run()
        plans[i % len(plans)][0].run()
    c.record()
    torch.cuda.synchronize()
    q_us = a.elapsed_time(b) / steps * 1e3
    step_us = b.elapsed_time(c) / steps * 1e3
    for p, _ in plans:
        p.free()
    qplan.free()
    # the plain streaming read of the quantiser's input bytes (h and g), every shape, timed the same way
    read_bytes = int(sum(8 * c[4] for c in ds.shapes))
    buf = torch.zeros(read_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    probe = {}
    for sh in range(bpw.PROBE_SHAPES):
        settle(torch, lambda: bpw.bpw_stream_read_probe(buf, sink, shape=sh))
        a.record()
        for i in range(steps):
            bpw.bpw_stream_read_probe(buf, sink, shape=sh)
        b.record()
        torch.cuda.synchronize()
        probe[str(sh)] = round(a.elapsed_time(b) / steps * 1e3, 2)
    return {"quantise_us": round(q_us, 2), "decode_step_with_quantise_us": round(step_us, 2),
            "quantised_values": int(sum(c[4] for c in ds.shapes)),
            "probe_same_read_bytes": {"bytes": read_bytes, "us_per_shape": probe, "best_us": min(probe.values())}}


def intmlp_measure(bpw, torch, dev, ds, steps: int = 100) -> dict:
    """The decode step with the MLP's squared-ReLU stage fused into gate/up: per layer q, k, v, o and
    down stay plain GEMVs and gate/up become one IntMlp pair reading the gate's activation, writing
    t = relu(a_g)^2 * a_u (int64) and K instead of the two projections' outputs. Same 521 MB of
    planes, one launch per step, the HBM copies in rotation, timed between HIP events."""
    ts, ks, plans = {}, {}, []
    for _, mats, _ in ds.copies:
        jobs, pairs = [], []
        for i, (layer, proj, name, rows, cols) in enumerate(ds.shapes):
            if proj == 5:
                continue
            x, s = ds.xs[i]
            if proj == 4:
                if layer not in ts:
                    ts[layer] = torch.empty(rows, dtype=torch.int64, device=dev)
                    ks[layer] = torch.empty(1, dtype=torch.float64, device=dev)
                pairs.append(bpw.intmlp_job(mats[i], mats[i + 1], x, s, ts[layer], ks[layer]))
            else:
                oi, of = ds.outs[i]
                jobs.append(bpw.gemv_job(mats[i], x, s, oi, of))
        ws = torch.empty(bpw.bpw_gemv_intmlp_workspace_bytes(jobs, pairs), dtype=torch.uint8, device=dev)
        plans.append((bpw.GemvPlan(jobs, ws, mlp=pairs), ws))
    def some():
        for i in range(10):
            plans[i % len(plans)][0].run()
    settle(torch, some)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        plans[i % len(plans)][0].run()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    for p, _ in plans:
        p.free()
    return {"decode_step_intmlp_us": round(us, 2), "weight_gbs": round(ds.plane_bytes / (us * 1e-6) / 1e9, 1),
            "pairs": len(ts), "plain_jobs": len(ds.shapes) - 2 * len(ts)}


def bitcos_measure(bpw, torch, dev, ds, steps: int = 100) -> dict:
    """The same 210 matrices re-encoded as BITCOS (presence bitmap + compacted signs, from the .trit
    host copies), in as many HBM copies as the .trit set, one grouped launch per step, timed between
    HIP events. Bytes: presence words, sign words and row_start words the launch reads."""
    plans, nbytes, sign_bytes, nnz = [], 0, 0, 0
    hosts = [bpw.bpw_bitcos_from_planes(hm) for hm in ds.host_mats]
    for h in hosts:
        p, s, r, k = h.arrays()
        nbytes += p.nbytes + s.nbytes + r.nbytes
        sign_bytes += s.nbytes
        nnz += k
    for _ in ds.copies:
        mats, bufs = [], []
        for h in hosts:
            buf = torch.empty(h.device_bytes, dtype=torch.uint8, device=dev)
            mats.append(bpw.bpw_bitcos_upload(h, buf))
            bufs.append(buf)
        jobs = [bpw.bitcos_job(m, x, s, oi, of) for m, (x, s), (oi, of) in zip(mats, ds.xs, ds.outs)]
        ws = torch.empty(bpw.bpw_bitcos_workspace_bytes(jobs), dtype=torch.uint8, device=dev)
        plans.append((bpw.BitcosPlan(jobs, ws), bufs, ws))
    for h in hosts:
        h.free()

    def some():
        for i in range(10):
            plans[i % len(plans)][0].run()
    settle(torch, some)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        plans[i % len(plans)][0].run()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1e3
    for p, _, _ in plans:
        p.free()
    gbs = nbytes / (us * 1e-6) / 1e9
    out = {"decode_step_bitcos_us": round(us, 2), "bytes": nbytes, "sign_bytes": sign_bytes, "nnz": nnz,
           "bits_per_weight": round(8.0 * nbytes / ds.weights, 4), "gbs": round(gbs, 1),
           "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2), "trit_plane_bytes": ds.plane_bytes}
    insts = bitcos_valu_from_profile()
    out["roofline"] = {
        "bound": "alu",
        "achieved": None if insts is None else round(insts * 64 / (us * 1e-6) / 1e12, 2),
        "peak": round(VALU_PEAK_LANE_OPS / 1e12, 2),
        "unit": "T int32 VALU lane-ops/s",
        "frac": None if insts is None else round(insts * 64 / (us * 1e-6) / VALU_PEAK_LANE_OPS, 4),
        "valu_insts_per_launch": insts,
        "kernel": "gemv_bitcos_kernel",
    }
    return out


def bitcos_valu_from_profile() -> float | None:
    """VALU wave-instructions per BITCOS decode-step launch from the committed counter run, if it was
    taken on the current kernel source; otherwise None."""
    try:
        with open(BITCOS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash(BITCOS_SRCS):
        return None
    return rec.get("sq_insts_valu_per_launch")


def configs_measure(bpw, torch, dev, ds, reps: int = 30) -> dict:
    """The smaller configurations of the same workload, timed the pages' way: HIP events around each
    launch, median and min over `reps`; hot = launches back to back (the weights stay in L2 and the
    last-level cache), cold = a 1 GiB read-modify-write flush before each timed launch (the flush is
    outside the timed span).
      k_proj: one 640 x 2560 matrix, 409,600 plane bytes (launch-latency dominated);
      layer: one layer's seven projections as one grouped launch (17,367,040 B), and each alone;
      decode step as 210 single-matrix launches in stream order, for context beside the grouped one;
      probe_same_bytes: the plain streaming read (every shape) of the k_proj's and the layer's bytes."""
    mats = ds.copies[0][1]

    def plan(idx):
        jobs = []
        for i in idx:
            x, s = ds.xs[i]
            oi, of = ds.outs[i]
            jobs.append(bpw.gemv_job(mats[i], x, s, oi, of))
        ws = torch.empty(bpw.bpw_gemv_workspace_bytes(jobs), dtype=torch.uint8, device=dev)
        return bpw.GemvPlan(jobs, ws), ws

    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def timed(fn, cold):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        settle(torch, fn)
        for a, b in ev:
            if cold:
                bpw.bpw_cache_flush(flush_buf)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        return statistics.median(t), t[0]

    def entry(nbytes, fn):
        out = {"bytes": nbytes}
        for kind in ("hot", "cold"):
            med, best = timed(fn, kind == "cold")
            out[kind] = {"us": round(med, 2), "min_us": round(best, 2), "gbs": round(nbytes / (med * 1e-6) / 1e9, 1)}
        return out

    layer0 = [i for i, sh in enumerate(ds.shapes) if sh[0] == 0]
    k_idx = [i for i in layer0 if ds.shapes[i][2] == "k_proj"]
    res = {}
    pk, _wk = plan(k_idx)
    res["k_proj_640x2560"] = entry(mats[k_idx[0]].rows * mats[k_idx[0]].bpr * 16, pk.run)
    pl, _wl = plan(layer0)
    layer_bytes = sum(mats[i].rows * mats[i].bpr * 16 for i in layer0)
    res["layer_grouped"] = entry(layer_bytes, pl.run)
    res["layer_per_matrix_hot_us"] = {}
    for i in layer0:
        p1, _w1 = plan([i])
        res["layer_per_matrix_hot_us"][ds.shapes[i][2]] = round(timed(p1.run, False)[0], 2)
        p1.free()
    singles = [plan([i]) for i in range(len(ds.shapes))]

    def step_singles():
        for p, _ in singles:
            p.run()
    med, best = timed(step_singles, False)
    res["decode_step_210_single_launches"] = {"us": round(med, 2), "min_us": round(best, 2),
                                              "gbs": round(ds.plane_bytes / (med * 1e-6) / 1e9, 1)}
    for p, _ in singles:
        p.free()

    def probe_entry(nbytes):
        # the plain streaming read of the same bytes, every shape, hot like the plans above: the floor
        # that a launch of this size reaches without any work of the method
        buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        per = {str(sh): round(timed(lambda: bpw.bpw_stream_read_probe(buf, sink, shape=sh), False)[0], 2)
               for sh in range(bpw.PROBE_SHAPES)}
        return {"bytes": nbytes, "hot_us_per_shape": per, "best_hot_us": min(per.values())}
    res["probe_same_bytes"] = {"k_proj_640x2560": probe_entry(res["k_proj_640x2560"]["bytes"]),
                               "layer_grouped": probe_entry(layer_bytes)}
    pk.free()
    pl.free()
    del flush_buf
    torch.cuda.empty_cache()
    return res


def probe_gbs(bpw, torch, dev) -> tuple[float, dict]:
    """Streaming-read probe (the pages' measured-roofline method): every read shape of the probe, best
    of 5 passes over 4 GiB each; the probe is the best shape. Returns (GB/s, GB/s per shape)."""
    n = 4 << 30
    buf = torch.zeros(n, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    per_shape = {}
    for shape in range(bpw.PROBE_SHAPES):
        settle(torch, lambda: bpw.bpw_stream_read_probe(buf, sink, shape=shape))
        best = 0.0
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            bpw.bpw_stream_read_probe(buf, sink, shape=shape)
            b.record()
            torch.cuda.synchronize()
            best = max(best, n / (a.elapsed_time(b) * 1e-3) / 1e9)
        per_shape[shape] = round(best, 1)
    del buf
    torch.cuda.empty_cache()
    return max(per_shape.values()), per_shape


def head_measure(bpw, torch, synth, dev, reps: int = 20) -> dict:
    """bf16 dense head 128256 x 2560 (two HBM copies in rotation), median over reps."""
    rows, cols = synth.VOCAB, synth.HIDDEN
    w, x = synth.head_case(BASE_SEED + 5)
    import numpy as np
    wd = [torch.from_numpy(w.view(np.int16)).to(dev) for _ in range(2)]
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    y = torch.empty(rows, dtype=torch.float32, device=dev)
    settle(torch, lambda: [bpw.bpw_dense_head_gemv(wd[i % 2], xd, y) for i in range(4)])
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record()
        bpw.bpw_dense_head_gemv(wd[i % 2], xd, y)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in ev)
    nbytes = rows * cols * 2
    return {"shape": [rows, cols], "bytes": nbytes, "us": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "pct_hbm_peak": 100.0 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def small_batch_measure(bpw, torch, synth, dev, reps: int = 64, kernel: int = 0) -> list[dict]:
    """Small-batch GEMM at gate/up (6912x2560) and down (2560x6912), B in 1..16; 64 rotating HBM
    copies of the matrix (283 MB) so weights come from HBM. One call is a few microseconds, less
    than the host needs to issue it, so `reps` calls (one per copy) are captured in a HIP graph and
    the graph replay is timed: per-call time = replay time / reps (kernel plus the gap between
    graph nodes)."""
    out = []
    for proj, rows, cols in ((4, 6912, 2560), (6, 2560, 6912)):
        case = synth.ternary_case(BASE_SEED + 7, 0, proj, rows, cols)
        hm = bpw.bpw_load(bpw.bpw_pack_i8(case.w), rows, cols, case.w_scale)
        mats, bufs = [], []
        for _ in range(64):
            buf = torch.empty(hm.nbytes, dtype=torch.uint8, device=dev)
            bufs.append(buf)
            mats.append(bpw.bpw_upload(hm, buf))
        nbytes = hm.nbytes
        hm.free()
        for batch in (1, 2, 4, 8, 16):
            X, sc = synth.small_batch_x(BASE_SEED + 11, batch, cols)
            Xd = torch.from_numpy(X).to(dev)
            oi = torch.empty((batch, rows), dtype=torch.int32, device=dev)
            of = torch.empty((batch, rows), dtype=torch.float32, device=dev)
            for i in range(3):
                bpw.bpw_gemm_small_batch(mats[i], Xd, sc, oi, of, kernel)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(reps):
                    bpw.bpw_gemm_small_batch(mats[i % 64], Xd, sc, oi, of, kernel)
            settle(torch, graph.replay, 20.0)
            times = []
            for _ in range(5):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                graph.replay()
                b.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b) / reps)
            ms = statistics.median(times)
            del graph
            out.append({"shape": [rows, cols], "batch": batch, "us": round(ms * 1e3, 2),
                        "weight_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "tops_equiv": round(2.0 * rows * cols * batch / (ms * 1e-3) / 1e12, 2)})
        del mats, bufs
    torch.cuda.empty_cache()
    return out


SB_RUNS = "1,2,2b,3,4,8,16"  # batch sizes of the grouped small-batch leg; "m" pins the matrix cores, "b" the
                             # bit-serial kernels (the token kernel from B = 2)


def grouped_small_batch_measure(bpw, torch, synth, dev, ds, steps: int = 50, runs_spec: str = SB_RUNS) -> list[dict]:
    """The decode-step set (210 matrices, 521 MB of planes) at batch B: every matrix times its own B
    int8 activation vectors, all in one grouped launch, the HBM copies in rotation. Under AUTO, B = 1
    runs the batch-1 GEMV and larger B the int8 matrix cores; B = 2 is also timed on the bit-serial
    token kernel (each beat streamed once, reduced against every token on the VALU). Shows where the
    weight stream stops being the limit as B grows."""
    out = []
    pin = {"m": bpw.KERNEL_MFMA, "b": bpw.KERNEL_BITSERIAL}
    runs = [(int(r.rstrip("mb")), pin.get(r[-1], bpw.KERNEL_AUTO)) for r in runs_spec.split(",")]
    names = {bpw.KERNEL_AUTO: "auto", bpw.KERNEL_MFMA: "mfma", bpw.KERNEL_BITSERIAL: "bitserial"}
    for batch, kernel in runs:
        xs = []
        for i, (layer, proj, name, rows, cols) in enumerate(ds.shapes):
            X, sc = synth.small_batch_x(BASE_SEED + 1009 * i + batch, batch, cols)
            xs.append((torch.from_numpy(X).to(dev), sc, torch.empty((batch, rows), dtype=torch.int32, device=dev),
                       torch.empty((batch, rows), dtype=torch.float32, device=dev)))
        plans = []
        for _, mats, _ in ds.copies:
            jobs = [bpw.sb_job(m, X, sc, oi, of) for m, (X, sc, oi, of) in zip(mats, xs)]
            ws = torch.empty(bpw.bpw_gemm_small_batch_workspace_bytes(jobs, batch), dtype=torch.uint8, device=dev)
            plans.append((bpw.SmallBatchPlan(jobs, batch, ws, kernel), ws))
        settle(torch, lambda: [plans[i % len(plans)][0].run() for i in range(6)])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            plans[i % len(plans)][0].run()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / steps * 1e3
        out.append({"batch": batch, "kernel": names[kernel], "us": round(us, 2),
                    "weight_gbs": round(ds.plane_bytes / (us * 1e-6) / 1e9, 1),
                    "tops_equiv": round(2.0 * ds.weights * batch / (us * 1e-6) / 1e12, 2)})
        for p, _ in plans:
            p.free()
        del plans, xs
    return out


def z_sweep_measure(bpw, torch, synth, dev, reps: int = 30) -> list[dict]:
    """Decode-step-shaped sets (one generated layer repeated over 30 layers, 2 HBM copies) at
    P(0) in the sweep; GEMV kernel median per step."""
    out = []
    for z in synth.P_ZERO_SWEEP:
        ds = DecodeSet(bpw, torch, synth, dev, copies=2, p_zero=z, base=BASE_SEED + 13, layers=lambda l: 0)
        settle(torch, lambda: [ds.plan(i).run() for i in range(10)])
        ms = statistics.median(time_steps(torch, ds, reps)[0] for _ in range(3))
        out.append({"p_zero": z, "gemv_us": round(ms * 1e3, 2),
                    "weight_gbs": round(ds.plane_bytes / (ms * 1e-3) / 1e9, 1)})
        ds.free_host()
        del ds
        torch.cuda.empty_cache()
    return out


CPU_LAYERS = 4  # decode-step layers in the CPU oracle's sample of the full step
CPU_HEAD_ROWS = 8192  # rows of the dense head in its CPU sample


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: the model name, then vendor, family, model and stepping
    numbers (a virtualised host may report only a generic model name such as "AMD EPYC")."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block is enough
                key, _, val = line.partition(":")
                fields.setdefault(key.strip(), val.strip())
    except OSError:
        return "unknown"
    ident = ", ".join(f"{k} {fields[k]}" for k in ("vendor_id", "cpu family", "model", "stepping") if k in fields)
    name = fields.get("model name", "unknown")
    return f"{name} ({ident})" if ident else name


def _median_rate(run, nbytes: int, min_seconds: float, runs: int = 3) -> tuple[float, list[float], float]:
    """`runs` timed runs, each repeating run() (nbytes per call) until min_seconds have passed.
    Returns (median GB/s, the per-run GB/s, total seconds)."""
    rates, total = [], 0.0
    for _ in range(runs):
        seconds, done = 0.0, 0
        while seconds < min_seconds:
            t = time.perf_counter()
            run()
            seconds += time.perf_counter() - t
            done += nbytes
        rates.append(done / seconds / 1e9)
        total += seconds
    return statistics.median(rates), rates, total


def cpu_baseline(cases, nthreads: int) -> dict:
    """The CPU oracle, as it is, on the host cores: the one-matrix case (the k projection of layer 0,
    640 x 2560), one layer (layer 0's seven projections), a sample of the decode step (its first
    CPU_LAYERS layers) and the bf16 head (its first CPU_HEAD_ROWS rows). Each is the median of three
    runs, in plane (or weight) GB/s; `value` is the decode-step sample's rate."""
    import numpy as np
    import oracle
    import synth

    packed = [(layer, oracle.pack(c.w), c) for layer, c in cases]

    def gemvs(items, threads):
        def run():
            for _, planes, c in items:
                oracle.gemv(planes, c.rows, c.cols, c.x, c.x_scale, c.w_scale, nthreads=threads)
        return run, sum(p.size for _, p, _ in items)

    layer0 = [t for t in packed if t[0] == 0]
    kproj = [t for t in layer0 if (t[2].rows, t[2].cols) == (640, 2560)][:1]
    out, seconds = {}, 0.0
    for name, items, min_s in (("k_proj_640x2560", kproj, 0.5), ("one_layer", layer0, 1.0),
                               (f"decode_step_first_{CPU_LAYERS}_layers", packed, 1.0)):
        run, nbytes = gemvs(items, nthreads)
        med, rates, sec = _median_rate(run, nbytes, min_s)
        seconds += sec
        out[name] = {"gbs": round(med, 4), "runs_gbs": [round(r, 4) for r in rates], "plane_bytes": nbytes,
                     "matrices": len(items)}
    w, x = synth.head_case(BASE_SEED + 5, rows=CPU_HEAD_ROWS)
    med, rates, sec = _median_rate(lambda: oracle.dense_head(w, x, nthreads=nthreads), w.nbytes, 1.0)
    seconds += sec
    out["dense_head_bf16"] = {"gbs": round(med, 4), "runs_gbs": [round(r, 4) for r in rates],
                              "weight_bytes": int(w.nbytes), "rows": CPU_HEAD_ROWS, "cols": int(w.shape[1])}
    run, nbytes = gemvs(layer0, 1)
    single, _, sec = _median_rate(run, nbytes, 1.0, runs=1)
    seconds += sec
    step = out[f"decode_step_first_{CPU_LAYERS}_layers"]
    return {
        "value": step["gbs"],
        "unit": "GB/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": f"the first {CPU_LAYERS} layers of the decode-step set ({step['matrices']} matrices, "
                  f"{step['plane_bytes']} plane bytes), one oracle GEMV per matrix on {nthreads} host threads, "
                  f"median of three runs; also the one-matrix and one-layer cases and the head's first "
                  f"{CPU_HEAD_ROWS} rows, {seconds:.1f} s of oracle time in all",
        "median_of": 3,
        "configs": out,
        "single_thread_one_layer_gbs": round(single, 4),
        "cpu_model": cpu_model(),
        "nproc": os.cpu_count(),
        "cpus_available": len(os.sched_getaffinity(0)),
    }


def traffic_from_profile() -> float | None:
    """HBM bytes per GEMV launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def _counter_rows(run_dir: str) -> list[dict]:
    """Rows of the rocprofv3 counter CSV (--output-format csv) under run_dir."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {run_dir}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _per_dispatch(rows: list[dict], kernel: str, counter: str, grid: int | None = None) -> list[float]:
    """Per-dispatch totals of one counter for the dispatches of one kernel (and grid size, in threads)."""
    acc: dict = {}
    for r in rows:
        if kernel not in r["Kernel_Name"] or r["Counter_Name"] != counter:
            continue
        if grid is not None and int(r["Grid_Size"]) != grid:
            continue
        acc[r["Dispatch_Id"]] = acc.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(acc.values())


def write_counter_records(fetch_dir: str, write_dir: str, bitcos_dir: str, out_gemv: str = TRAFFIC_FILE,
                          out_bitcos: str = BITCOS_FILE) -> None:
    """Write the two committed counter records from three rocprofv3 runs of this file, each with
    --copy-calibration --legs bitcos: FETCH_SIZE, WRITE_SIZE, and the BITCOS kernel's SQ counters
    (SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAVES). Byte counters are scaled by what they
    read for the copy calibration (the probe reads 1 GiB, the flush rewrites 1 GiB); each figure is the
    median over the dispatches. The records carry the hash of the kernel sources as they are now."""
    fr, wr, br = _counter_rows(fetch_dir), _counter_rows(write_dir), _counter_rows(bitcos_dir)
    gib_kib = float(1 << 20)
    probe_fetch = statistics.median(_per_dispatch(fr, "stream_probe_kernel", "FETCH_SIZE"))
    flush_write = statistics.median(_per_dispatch(wr, "flush_kernel", "WRITE_SIZE"))
    fetch_scale, write_scale = gib_kib / probe_fetch, gib_kib / flush_write
    cal = (f"FETCH_SIZE of the streaming probe reading 1 GiB ({gib_kib:.0f} KiB) read {probe_fetch:.1f} KiB; "
           f"WRITE_SIZE of the cache flush rewriting 1 GiB read {flush_write:.1f} KiB")
    steps = 11712 * 256  # the decode-step launch's grid, in threads
    gf = statistics.median(_per_dispatch(fr, "gemv_bitserial_kernel", "FETCH_SIZE", steps))
    gw = statistics.median(_per_dispatch(wr, "gemv_bitserial_kernel", "WRITE_SIZE", steps))
    rel = lambda paths: [os.path.relpath(q, ROOT) for q in paths]  # noqa: E731
    gemv = {
        "kernel": "gemv_bitserial_kernel",
        "workload": "decode-step ternary GEMV set, 210 matrices, 521011200 plane bytes, batch 1",
        "kernel_source_sha256": kernel_source_hash(),
        "kernel_sources": rel(KERNEL_SRCS),
        "fetch_size_kib_per_dispatch": round(gf, 1),
        "write_size_kib_per_dispatch": round(gw, 1),
        "fetch_scale": round(fetch_scale, 5),
        "write_scale": round(write_scale, 5),
        "calibration": cal,
        "traffic_bytes_per_launch": int(round(gf * 1024 * fetch_scale + gw * 1024 * write_scale)),
        "algorithmic_bytes_per_launch": {"planes": 521011200, "activations": 668160, "outputs_i32_f32": 5468160},
    }
    bf = statistics.median(_per_dispatch(fr, "gemv_bitcos_kernel", "FETCH_SIZE"))
    bw = statistics.median(_per_dispatch(wr, "gemv_bitcos_kernel", "WRITE_SIZE"))
    sq = {c: statistics.median(_per_dispatch(br, "gemv_bitcos_kernel", c))
          for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES")}
    bitcos = {
        "kernel": "gemv_bitcos_kernel",
        "workload": "decode-step ternary GEMV set as BITCOS, 210 matrices, 415166556 bytes (presence 260505600, "
                    "sign words 151926036, row_start 2734920), batch 1",
        "kernel_source_sha256": kernel_source_hash(BITCOS_SRCS),
        "kernel_sources": rel(BITCOS_SRCS),
        "sq_insts_valu_per_launch": int(sq["SQ_INSTS_VALU"]),
        "sq_insts_lds_per_launch": int(sq["SQ_INSTS_LDS"]),
        "sq_lds_bank_conflict_cycles_per_launch": int(sq["SQ_LDS_BANK_CONFLICT"]),
        "sq_waves_per_launch": int(sq["SQ_WAVES"]),
        "fetch_size_kib_per_dispatch": round(bf, 1),
        "write_size_kib_per_dispatch": round(bw, 1),
        "fetch_scale": round(fetch_scale, 5),
        "write_scale": round(write_scale, 5),
        "traffic_bytes_per_launch": int(round(bf * 1024 * fetch_scale + bw * 1024 * write_scale)),
        "algorithmic_bytes_per_launch": {"presence": 260505600, "sign_words": 151926036, "row_start": 2734920,
                                         "activations": 668160, "outputs_i32_f32": 5468160},
    }
    for path, rec in ((out_gemv, gemv), (out_bitcos, bitcos)):
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        log(f"wrote {os.path.relpath(path, ROOT)}: {rec['traffic_bytes_per_launch']} bytes per launch")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first (the clocks need about 250 decode steps, ~20 ms, to ramp up)")
    ap.add_argument("--copies", type=int, default=3, help="HBM copies of the weight set used in rotation")
    ap.add_argument("--kernel", choices=("auto", "bitserial", "bytelane"), default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip every companion measurement")
    ap.add_argument("--legs", default="all",
                    help="comma-separated companion measurements to run (default all): " + ",".join(LEGS))
    ap.add_argument("--sb-batches", default=SB_RUNS,
                    help="batch sizes of the small_batch_decode_step leg, comma-separated; a trailing m pins the "
                         "matrix cores, a trailing b the bit-serial kernels (default %(default)s)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the steps, read 1 GiB with the streaming probe and rewrite 1 GiB with the cache "
                         "flush (3 times each): kernels of known traffic for scaling hardware byte counters")
    ap.add_argument("--write-counter-records", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "BITCOS_SQ_DIR"),
                    help="no GPU: write the committed counter records from three rocprofv3 counter runs of this "
                         "file (see write_counter_records) and exit")
    args = ap.parse_args()
    if args.write_counter_records:
        write_counter_records(*args.write_counter_records)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import numpy as np  # noqa: F401
    import torch

    import bit_plane_weight_amd as bpw
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bpw.bpw_device_check()
    kernel = {"auto": bpw.KERNEL_AUTO, "bitserial": bpw.KERNEL_BITSERIAL, "bytelane": bpw.KERNEL_BYTELANE}[args.kernel]

    # ---------------------------------------------------------------- CPU oracle baseline (host cores)
    nthreads = host_threads()
    sample = []
    oracle_fn = None
    if not args.no_cpu_baseline:
        def oracle_fn(case, layer):
            if layer < CPU_LAYERS:
                sample.append((layer, case))

    log("generating, packing and uploading the decode-step set")
    t0 = time.perf_counter()
    ds = DecodeSet(bpw, torch, synth, dev, copies=args.copies, p_zero=synth.P_ZERO_2B4T, base=BASE_SEED,
                   cpu_oracle=oracle_fn)
    if kernel != bpw.KERNEL_AUTO:
        for i, (plan, mats, ws) in enumerate(ds.copies):
            plan.free()
            jobs = [bpw.gemv_job(m, x, s, oi, of) for m, (x, s), (oi, of) in zip(mats, ds.xs, ds.outs)]
            ds.copies[i] = (bpw.GemvPlan(jobs, ws, kernel), mats, ws)
    log(f"setup {time.perf_counter() - t0:.1f}s: {ds.weights} weights, {ds.plane_bytes} plane bytes, "
        f"{len(ds.copies)} copies")

    # ---------------------------------------------------------------- timed steps
    for i in range(args.warmup):
        ds.plan(i).run()
    torch.cuda.synchronize()
    K = args.steps
    # timed region: K back-to-back steps, a barrier (device synchronisation) on both sides
    kern_avg_ms, ms_per_step = time_steps(torch, ds, K)
    value = ds.plane_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = ds.plane_bytes / (kern_avg_ms * 1e-3) / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us wall, {value:.0f} GB/s; GEMV launch avg {kern_avg_ms * 1e3:.1f} us "
        f"(HIP events), {achieved:.0f} GB/s")

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i32",
        "data": "synthetic",
        "config": {
            "workload": "decode-step ternary GEMV set: 210 .trit v1 matrices (30 layers x q 2560x2560, "
                        "k/v 640x2560, o 2560x2560, gate/up 6912x2560, down 2560x6912), BitNet b1.58 2B4T "
                        "shapes, batch 1, int8 absmax activations, P(0)=0.4219, weights streamed from HBM",
            "matrices": 210,
            "weights": ds.weights,
            "plane_bytes": ds.plane_bytes,
            "hbm_copies_in_rotation": len(ds.copies),
            "kernel": args.kernel,
        },
        "decode_step_us": round(ms_per_step * 1e3, 2),
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(),
            "kernel": "gemv_bitserial_kernel" if kernel != bpw.KERNEL_BYTELANE else "gemv_bytelane_kernel",
            "kernel_avg_us": round(kern_avg_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": ds.plane_bytes,
        },
    }
    if sample:
        log("CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(sample, nthreads)

    if args.copy_calibration:
        log("copy calibration: probe reads 1 GiB, flush reads and writes 1 GiB, 3 times each")
        cal = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(3):
            bpw.bpw_stream_read_probe(cal, sink)
        for _ in range(3):
            bpw.bpw_cache_flush(cal)
        torch.cuda.synchronize()
        del cal

    # ---------------------------------------------------------------- companion measurements
    legs = set() if args.no_extras else (set(LEGS) if args.legs == "all" else set(args.legs.split(",")))
    unknown = legs - set(LEGS)
    if unknown:
        print(f"unknown --legs {sorted(unknown)}; choose from {','.join(LEGS)}", file=sys.stderr)
        return 2
    if "configs" in legs:
        log("k_proj, one layer (hot and cold), 210 single launches")
        result["configs"] = configs_measure(bpw, torch, dev, ds)
    if "prologue" in legs:
        log("quantiser prologue")
        result["prologue"] = prologue_measure(bpw, torch, synth, dev, ds)
    if "intmlp" in legs:
        log("IntMlp pairs")
        result["intmlp"] = intmlp_measure(bpw, torch, dev, ds)
    if "small_batch_decode_step" in legs:
        log("grouped small batch over the decode-step set")
        result["small_batch_decode_step"] = grouped_small_batch_measure(bpw, torch, synth, dev, ds,
                                                                        runs_spec=args.sb_batches)
    if "bitcos" in legs:
        log("BITCOS decode step")
        result["bitcos"] = bitcos_measure(bpw, torch, dev, ds)
        result["bitcos"]["vs_trit_step"] = round(result["bitcos"]["decode_step_bitcos_us"] / (kern_avg_ms * 1e3), 3)
    ds.free_host()
    ds = None
    torch.cuda.empty_cache()
    if "probe" in legs:
        log("probe")
        pg, shapes = probe_gbs(bpw, torch, dev)
        result["probe_gbs"] = round(pg, 1)
        result["probe_gbs_per_shape"] = shapes
        result["pct_probe"] = round(100.0 * achieved / pg, 2)
    if "head" in legs:
        log("dense head")
        head = head_measure(bpw, torch, synth, dev)
        result["head"] = {k: (round(v, 2) if isinstance(v, float) else v) for k, v in head.items()}
        result["per_token_us"] = round(kern_avg_ms * 1e3 + head["us"], 2)
        result["per_token_bytes"] = result["config"]["plane_bytes"] + head["bytes"]
    if "z_sweep" in legs:
        log("zero-density sweep")
        result["z_sweep"] = z_sweep_measure(bpw, torch, synth, dev)
    if "small_batch" in legs:
        log("small batch")
        result["small_batch"] = small_batch_measure(bpw, torch, synth, dev)  # auto: the matrix-core kernel
        result["small_batch_bitserial"] = small_batch_measure(bpw, torch, synth, dev, kernel=bpw.KERNEL_BITSERIAL)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
