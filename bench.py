"""Benchmark of the emulated-rank AllReduce on one MI355X.

Default run (one JSON line on stdout):
  * value: microseconds per reduce of the AUTO protocol on N = 8 emulated
    ranks x 16 KiB bf16 (8192 elements per rank), inputs resident in HBM.
    After --warmup untimed calls, exactly --steps calls are timed with HIP
    events on the launch stream, once back to back and once replayed from a
    HIP graph of those calls; the faster is `value`, both are reported with
    the number of calls each timed region held;
  * latency: the same reduce measured device-side (first workgroup start to
    last workgroup end) against the single-GPU speed-of-light floor
    2 x (L2 round trip) + (cross-XCD store visibility), all measured here,
    with the L2 round trip also to lines another XCD has just written and
    the empty-launch interval both plain and graph-replayed;
  * bandwidth_64MiB: the 64 MiB-per-rank reduce, effective GB/s over the
    algorithmic bytes (N + 1) x 64 MiB, and the HBM roofline of that kernel;
  * sweep: the AUTO protocol at 128 B .. 64 MiB per rank (20 sizes) and the
    least-squares fit T(size) = alpha + beta * size (the pwwt.cn
    small-message latency article, section 2.1), overall and per protocol;
  * atomic_ceiling and the LL128 workload rows: the measured throughput of
    device-scope float atomics with the LL128 lane pattern, and the LL128
    kernels' atomic lane operations per second against it;
  * barrier_ablation: the same 16 KiB one-shot reduce with a grid-wide
    barrier in place of the LL flags, beside LL itself;
  * rows: send/recv (8 KB fp16), ReduceScatter / AllGather at N = 8, 16 KiB;
  * cpu_baseline: the CPU oracle on the same 16 KiB workload, on one host
    thread and on every host core; this leg also compares the GPU outputs
    kept from the timed runs with the oracle (output_check).

--sweep-all adds every protocol's sweep (written to --sweep-out).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per reduce (16 KB bf16, N=8) vs SoL floor; GB/s at 64 MB"
HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
N_RANKS = 8
SMALL_BYTES = 16 << 10
BIG_BYTES = 64 << 20
TRAFFIC_PROFILE = "sentinel_pipelined_64MiB_x8_bf16.pmc.txt"
PROTO_NAMES = {0: "auto", 1: "ll", 2: "sentinel", 3: "ll128", 4: "ll128_pipelined", 5: "sentinel_pipelined"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fit_alpha_beta(sizes, times):
    """Least-squares fit of T(size) = alpha + beta * size (the pwwt.cn
    small-message latency article, section 2.1: a fixed start-up cost plus
    a per-byte cost)."""
    x = np.asarray(sizes, dtype=np.float64)
    y = np.asarray(times, dtype=np.float64)
    a = np.vstack([np.ones_like(x), x]).T
    (alpha, beta), *_ = np.linalg.lstsq(a, y, rcond=None)
    return float(alpha), float(beta)


def graph_split(steps, cap=1000):
    """(calls per graph, replays) with calls x replays == steps exactly and
    at most `cap` calls captured in one graph."""
    steps = max(1, int(steps))
    per = max(d for d in range(1, min(steps, cap) + 1) if steps % d == 0)
    return per, steps // per


def device_inputs(cfg_id, n_ranks, n, dist, scale, rep=0):
    import torch
    from workloads import make_partials
    bits = make_partials(cfg_id, rep, n_ranks, "bf16", n, dist, scale)
    parts = [torch.from_numpy(bits[r].view(np.int16).copy()).view(torch.bfloat16).cuda() for r in range(n_ranks)]
    return bits, parts


def order_after_current(stream):
    """Make `stream` wait for the work already queued on the caller's current
    stream.  Inputs and outputs are made there, and the caching allocator may
    hand an output a block whose previous user (say, a dtype conversion's
    temporary) is still being read there: without this order a call on
    `stream` could write that block under the pending reader."""
    import torch
    stream.wait_stream(torch.cuda.current_stream())


def time_calls(comm, parts, out, proto, steps, warmup, stream):
    """Per-call microseconds of `steps` back-to-back calls (HIP events on the
    launch stream), after `warmup` untimed calls."""
    import torch
    order_after_current(stream)
    call = comm.prepare(parts, out, proto, stream=stream)
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            call()
        b.record(stream)
        torch.cuda.synchronize()
    st, bits = comm.device_status()
    if st != 0:
        raise RuntimeError("device status %d (bits %#x) during %s" % (st, bits, proto))
    return a.elapsed_time(b) * 1e3 / steps


def time_batches(comm, parts, out, proto, steps, warmup, stream, batches=5):
    """Per-call microseconds in `batches` timed batches of steps/batches
    calls each: (min, median, p90) over the batches."""
    per = max(1, steps // batches)
    xs = sorted(time_calls(comm, parts, out, proto, per, warmup if i == 0 else 0, stream) for i in range(batches))
    return xs[0], statistics.median(xs), xs[min(len(xs) - 1, int(round(0.9 * (len(xs) - 1))))]


def time_graph(comm, parts, out, proto, steps, stream):
    """Per-call microseconds of exactly `steps` calls captured into HIP
    graphs (at most 1000 calls per graph) and replayed: the launch cost a
    captured decode step pays.  Captured calls read the device-resident
    epoch, so every replay is a fresh call."""
    import torch
    order_after_current(stream)
    call = comm.prepare(parts, out, proto, stream=stream)
    per_graph, reps = graph_split(steps)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        call()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(per_graph):
                call()
        torch.cuda.synchronize()
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    st, bits = comm.device_status()
    if st != 0:
        raise RuntimeError("device status %d (bits %#x) during graph replay of %s" % (st, bits, proto))
    del g
    return a.elapsed_time(b) * 1e3 / (reps * per_graph)


def time_graph_fn(fn, steps, stream, per_graph=100):
    """Per-call microseconds of `fn` (one library call on `stream`) from
    replays of a HIP graph of `per_graph` captured calls: GPU time only, no
    Python call overhead."""
    import torch
    order_after_current(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(per_graph):
                fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // per_graph)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) * 1e3 / (reps * per_graph)


def device_side_fn(comm, fn, calls, stream):
    """Median and minimum device-side microseconds of `fn` (first workgroup
    start to last workgroup end) over `calls` calls."""
    import torch
    order_after_current(stream)
    import message_allreduce_amd as llar
    calls = min(calls, 60)
    comm.set_option("timing", 1)
    try:
        with torch.cuda.stream(stream):
            for _ in range(calls):
                fn()
        torch.cuda.synchronize()
        recs = comm.timing(calls)
    finally:
        comm.set_option("timing", 0)
    hz = llar.llar_wallclock_hz()
    d = sorted((t1 - t0) / hz * 1e6 for t0, t1 in recs if t1 > t0)
    return statistics.median(d), d[0]


def measure_rows(stream, steps):
    """The other collectives at the shapes the pages give them: point-to-point
    send/recv of one token's 4096 x fp16 hidden state (8 KB) between two
    pipeline stages, and ReduceScatter / AllGather of the N = 8, 16 KiB bf16
    tensor-parallel hidden state (2 KiB segments)."""
    import torch
    import message_allreduce_amd as llar
    rows = {}
    # the pages' smallest case: two ranks, 128 bytes of fp32, LL one-shot
    c1 = llar.Communicator(2, torch.float32, 128)
    try:
        p1 = [torch.randn(32, dtype=torch.float32, device="cuda") for _ in range(2)]
        o1 = torch.empty(32, dtype=torch.float32, device="cuda")
        fn = (lambda: c1.allreduce(p1, o1, "ll", stream=stream))
        us = time_graph_fn(fn, steps, stream)
        dmed, dmin = device_side_fn(c1, fn, 60, stream)
        rows["allreduce_128B_x2_fp32_ll"] = {"us_per_call_graph": round(us, 3), "device_us_median": round(dmed, 3),
                                             "device_us_min": round(dmin, 3)}
        log("allreduce 128 B x 2 fp32 ll: %.3f us per call (graph), device %.3f us" % (us, dmed))
        st, bits = c1.device_status()
        if st != 0:
            raise RuntimeError("device status %d (bits %#x) in the 128 B timing" % (st, bits))
    finally:
        c1.close()
    c2 = llar.Communicator(2, torch.float16, 8192)
    try:
        send = torch.randn(4096, dtype=torch.float16, device="cuda")
        recv = torch.empty_like(send)
        for wire in ("ll", "sentinel"):
            fn = (lambda w=wire: c2.send_recv(send, recv, w, stream=stream))
            us = time_graph_fn(fn, steps, stream)
            dmed, dmin = device_side_fn(c2, fn, 60, stream)
            rows["send_recv_8KB_fp16_" + wire] = {"us_per_call_graph": round(us, 3), "device_us_median": round(dmed, 3),
                                                  "device_us_min": round(dmin, 3)}
            log("send/recv 8 KB fp16 %s: %.3f us per call (graph), device %.3f us" % (wire, us, dmed))
        st, bits = c2.device_status()
        if st != 0:
            raise RuntimeError("device status %d (bits %#x) in send/recv timing" % (st, bits))
    finally:
        c2.close()
    c8 = llar.Communicator(N_RANKS, torch.bfloat16, SMALL_BYTES)
    try:
        n = SMALL_BYTES // 2
        cnt = n // N_RANKS
        _, parts = device_inputs(5, N_RANKS, n, "normal", 1.0)
        segs = [torch.empty(cnt, dtype=torch.bfloat16, device="cuda") for _ in range(N_RANKS)]
        full = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(N_RANKS)]
        for wire in ("ll", "sentinel", "ll128"):
            calls = [("reduce_scatter", lambda w=wire: c8.reduce_scatter(parts, segs, w, stream=stream))]
            if wire != "ll128":  # nothing to sum in an AllGather
                calls.append(("all_gather", lambda w=wire: c8.all_gather(segs, full, w, stream=stream)))
            for name, fn in calls:
                us = time_graph_fn(fn, steps, stream)
                dmed, dmin = device_side_fn(c8, fn, 60, stream)
                rows["%s_16KiB_x8_bf16_%s" % (name, wire)] = {"us_per_call_graph": round(us, 3),
                                                               "device_us_median": round(dmed, 3),
                                                               "device_us_min": round(dmin, 3)}
                log("%s 16 KiB x 8 bf16 %s: %.3f us per call (graph), device %.3f us" % (name, wire, us, dmed))
        st, bits = c8.device_status()
        if st != 0:
            raise RuntimeError("device status %d (bits %#x) in collective timing" % (st, bits))
    finally:
        c8.close()
    return rows


def measure_workloads(stream, steps, floor_us, ceiling, checks):
    """The four fixed workloads of the parity suite, each with its own
    protocol, rank count and dtype (the fifth is the size sweep): per call
    from graph replay, the device-side span, the span over the latency floor,
    and the algorithmic (N + 1) x S bytes over the span against the HBM peak.
    The LL128 rows add their atomic lane operations per second against the
    measured atomic ceiling of their staging type; workload 2 runs with both
    stagings (binary32, and the 16-bit packed lines of the page's FP16
    case).  Each row's output is kept for the oracle check."""
    import torch
    import message_allreduce_amd as llar
    from workloads import WORKLOADS, workload_partials
    tdt = {"fp32": (torch.float32, np.int32, 0), "fp16": (torch.float16, np.int16, 1),
           "bf16": (torch.bfloat16, np.int16, 2)}
    rows = {}
    runs = [(1, 0), (2, 0), (2, 1), (3, 0), (4, 0)]
    for k, acc16 in runs:
        w = WORKLOADS[k]
        dt, it, code = tdt[w.dtype]
        nbytes = w.n_elems * torch.tensor([], dtype=dt).element_size()
        c = llar.Communicator(w.n_ranks, dt, nbytes)
        name = w.name + ("_acc16" if acc16 else "")
        try:
            if w.chunk_bytes:
                c.set_option("chunk_bytes", w.chunk_bytes)
            if acc16:
                c.set_option("ll128_acc", 1)
            bits = workload_partials(w, 0)
            parts = [torch.from_numpy(bits[r].view(it).copy()).view(dt).cuda() for r in range(w.n_ranks)]
            out = torch.empty(w.n_elems, dtype=dt, device="cuda")
            fn = (lambda: c.allreduce(parts, out, w.protocol, stream=stream))
            # the 4 MiB pipelined workload takes ~0.25 ms per call: 500 calls
            us = time_graph_fn(fn, 500 if w.chunk_bytes else steps, stream)
            dmed, dmin = device_side_fn(c, fn, 60, stream)
            alg = (w.n_ranks + 1) * nbytes
            gbps = alg / dmed / 1e3
            row = {"protocol": w.protocol, "n_ranks": w.n_ranks, "dtype": w.dtype, "bytes_per_rank": nbytes,
                   "us_per_call_graph": round(us, 3), "device_us_median": round(dmed, 3),
                   "device_us_min": round(dmin, 3), "device_over_floor": round(dmed / floor_us, 3),
                   "GBps_device": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 5)}
            if w.protocol.startswith("ll128"):
                geo = c.geometry(w.n_elems, llar.PROTOCOLS[w.protocol])
                chunk = -(-w.n_elems // geo["chunks"])
                ops = ll128_lane_ops(w.n_ranks, w.n_elems, chunk, bool(acc16))
                reqs = ll128_requests(w.n_ranks, w.n_elems, chunk, bool(acc16))
                rate = ops / (dmed * 1e-6) / 1e9
                rreq = reqs / (dmed * 1e-6) / 1e9
                ceil = ceiling["pk_bf16_8way_cross_xcd" if acc16 else "f32_8way_cross_xcd"]
                # the microbenchmark's requests carry 16 lanes each (64 bytes;
                # TCC_ATOMIC counts 8 388 608 requests for its 134 M lanes)
                ceil_req = ceil / 16.0
                row.update({"staging": "16-bit packed" if acc16 else "binary32", "atomic_lane_ops": ops,
                            "atomic_G_lane_ops_per_s": round(rate, 2), "atomic_ceiling_G_per_s": ceil,
                            "frac_of_atomic_ceiling": round(rate / ceil, 4) if ceil else None,
                            "atomic_requests": reqs, "atomic_G_requests_per_s": round(rreq, 3),
                            "atomic_request_ceiling_G_per_s": round(ceil_req, 3),
                            "frac_of_atomic_request_ceiling": round(rreq / ceil_req, 4) if ceil else None})
            rows[name] = row
            log("workload %d %s: %.3f us per call (graph), device %.3f us, %.1f GB/s%s"
                % (k, name, us, dmed, gbps, "" if "atomic_G_lane_ops_per_s" not in row else
                   ", %.2f G atomic lane ops/s" % row["atomic_G_lane_ops_per_s"]))
            st, sbits = c.device_status()
            if st != 0:
                raise RuntimeError("device status %d (bits %#x) in workload %d" % (st, sbits, k))
            got = out.view(torch.int32 if code == 0 else torch.int16).cpu().numpy().view(
                np.uint32 if code == 0 else np.uint16)
            checks.append((name, bits, got, code, not w.protocol.startswith("ll128")))
        finally:
            c.close()
    return rows


def measure_device_api(stream, steps):
    """The device-side API's use case: an epilogue fused with the exchange.
    N = 8 fp32 partials of 16 KiB are scaled per rank and summed, either by
    one custom kernel written against include/llar_wire.h (the LL demo of
    tests/device_api) or by a scaling kernel followed by the library's LL
    AllReduce.  Per call from graph replay; None if the demo is not built."""
    import ctypes
    import torch
    import message_allreduce_amd as llar
    lib = os.path.join(ROOT, "tests", "device_api", "libwire_demo.so")
    if not os.path.exists(lib):
        return None
    L = ctypes.CDLL(lib)
    vp, u32, u64, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
    L.demo_scaled_allreduce_ll.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_float), vp, u32, i32, vp, u32,
                                           u32, u64, vp, vp]
    L.demo_scaled_allreduce_ll.restype = i32
    n = SMALL_BYTES // 4
    stacked = torch.randn(N_RANKS, n, dtype=torch.float32, device="cuda")
    scales = torch.linspace(0.5, 2.0, N_RANKS, dtype=torch.float32, device="cuda").view(N_RANKS, 1)
    scaled = torch.empty_like(stacked)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    stage = torch.zeros((N_RANKS - 1) * ((n + 1) // 2) * 16, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ptrs = (vp * N_RANKS)(*[stacked[r].data_ptr() for r in range(N_RANKS)])
    host_scales = (ctypes.c_float * N_RANKS)(*scales.view(-1).tolist())
    def fused(epoch):
        rc = L.demo_scaled_allreduce_ll(ptrs, host_scales, out.data_ptr(), n, N_RANKS, stage.data_ptr(),
                                        stage.numel(), epoch, 10_000_000, status.data_ptr(),
                                        ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("demo_scaled_allreduce_ll returned %d" % rc)

    # A captured launch repeats its arguments: the graph holds 100 launches
    # with epochs 1..100, and the LL staging is cleared (one fill kernel)
    # before each replay so that no line of the previous replay looks valid.
    order_after_current(stream)
    per_graph = 100
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        stage.zero_()
        fused(1)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for ep in range(1, per_graph + 1):
                fused(ep)
        torch.cuda.synchronize()
        stage.zero_()
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // per_graph)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            stage.zero_()
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    us_fused = a.elapsed_time(b) * 1e3 / (reps * per_graph)
    del g

    c = llar.Communicator(N_RANKS, torch.float32, SMALL_BYTES)
    try:
        parts = [scaled[r] for r in range(N_RANKS)]

        def unfused():
            torch.mul(stacked, scales, out=scaled)
            c.allreduce(parts, out, "ll", stream=stream)

        us_unfused = time_graph_fn(unfused, steps, stream, per_graph)
        torch.cuda.synchronize()
        if int(status.item()) != 0 or c.device_status()[0] != 0:
            raise RuntimeError("a wait expired in the device-API timing")
    finally:
        c.close()
    log("device API: fused scale+allreduce %.3f us per call, scale kernel + llar_allreduce %.3f us"
        % (us_fused, us_unfused))
    return {"workload": "8 x 16 KiB fp32 partials, per-rank scale then sum",
            "fused_us_per_call_graph": round(us_fused, 3),
            "unfused_us_per_call_graph": round(us_unfused, 3)}


def profiled_traffic(kernel_file, name):
    """HBM bytes per launch of the 64 MiB reduce, from the committed counter
    summary -- only while the kernel source is the one that was profiled."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None, None
    with open(kernel_file, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line)
    if fields.get("kernel_source_sha256", "").strip() != digest:
        return None, "kernel changed since %s was taken" % name
    return float(fields["traffic_bytes_per_launch"]), name


def device_side_us(comm, parts, out, proto, calls, stream):
    """Median device-side microseconds (first workgroup start to last
    workgroup end, wall clock) over `calls` timed calls."""
    import torch
    order_after_current(stream)
    import message_allreduce_amd as llar
    calls = min(calls, 60)
    comm.set_option("timing", 1)
    try:
        with torch.cuda.stream(stream):
            for _ in range(calls):
                comm.allreduce(parts, out, proto, stream=stream)
        torch.cuda.synchronize()
        recs = comm.timing(calls)
    finally:
        comm.set_option("timing", 0)
    hz = llar.llar_wallclock_hz()
    d = sorted((t1 - t0) / hz * 1e6 for t0, t1 in recs if t1 > t0)
    return statistics.median(d), d[0]


def measure_floor():
    import message_allreduce_amd as llar
    rt = statistics.median(llar.llar_floor_measure(0) for _ in range(3))
    stores = {}
    for b in range(1, 8):
        stores[b] = llar.llar_floor_measure(1, b)
    same_xcd = llar.llar_floor_measure(1, 8)
    t_store = statistics.mean(stores.values())
    launch = llar.llar_floor_measure(2)
    launch_graph = llar.llar_floor_measure(6, 100)
    atomic = llar.llar_floor_measure(3)
    # L2 round trip to lines another XCD has just written (a consumer's read
    # of a producer's store), and to lines another workgroup of XCD 0 wrote
    rt_written = {b: llar.llar_floor_measure(5, b) for b in range(1, 8)}
    rt_written_same = llar.llar_floor_measure(5, 8)
    rt_cross = statistics.mean(rt_written.values())
    floor_ns = 2 * rt + t_store
    return {
        "t_l2_round_trip_written_cross_xcd_ns": round(rt_cross, 1),
        "t_l2_round_trip_written_by_xcd_ns": {str(k): round(v, 1) for k, v in rt_written.items()},
        "t_l2_round_trip_written_same_xcd_ns": round(rt_written_same, 1),
        # the floor with the cross-XCD round trip in both terms (reported; the
        # floor the targets use keeps the smaller L2-hit round trip)
        "floor_cross_xcd_rt_us": round((2 * rt_cross + t_store) / 1e3, 4),
        "empty_launch_graph_us": round(launch_graph / 1e3, 3),
        "t_l2_round_trip_ns": round(rt, 1),
        "t_store_cross_xcd_ns": round(t_store, 1),
        "t_store_by_xcd_ns": {str(k): round(v, 1) for k, v in stores.items()},
        "t_store_same_xcd_ns": round(same_xcd, 1),
        "floor_us": round(floor_ns / 1e3, 4),
        "floor_same_xcd_us": round((2 * rt + same_xcd) / 1e3, 4),
        # the shorter reading of the same bound: one L2 round trip plus one store
        "floor_rt_plus_store_us": round((rt + t_store) / 1e3, 4),
        "empty_launch_us": round(launch / 1e3, 3),
        "atomic_latency_ns": round(atomic, 1),
    }


def host_cpu():
    """CPU model and the number of cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def cpu_baseline(seconds, checks):
    """The oracle as it stands, timed on the host on repeated reduces of the
    same 16 KiB x 8 bf16 input: on one thread, then on every core (one
    thread per core, each reducing whole messages; the C routine releases
    the interpreter lock).  Then the GPU outputs kept from the timed runs
    are compared with the oracle: `checks` holds (name, partial bits, GPU
    output bits, dtype, exact?)."""
    import concurrent.futures as cf
    import oracle
    from workloads import make_partials
    model, cores = host_cpu()
    bits = make_partials(5, 0, N_RANKS, "bf16", SMALL_BYTES // 2, "normal", 1.0)
    oracle.allreduce(bits, oracle.BF16)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds / 2:
        oracle.allreduce(bits, oracle.BF16)
        n += 1
    dt1 = time.perf_counter() - t0
    one = dt1 / n * 1e6

    def worker(deadline):
        k = 0
        while time.perf_counter() < deadline:
            oracle.allreduce(bits, oracle.BF16)
            k += 1
        return k

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        counts = list(ex.map(worker, [t0 + seconds / 2] * cores))
    dtn = time.perf_counter() - t0
    alln = dtn / sum(counts) * 1e6
    result = {"value": round(alln, 2), "unit": "us per reduce", "cores": cores, "kind": "oracle",
              "sample": "%d reduces of the 16 KiB x 8 bf16 workload in %.1f s on %d host threads (one per core); "
                        "throughput: wall time over reduces" % (sum(counts), dtn, cores),
              "cpu_model": model,
              "single_thread": {"value": round(one, 2), "unit": "us per reduce", "cores": 1,
                                "sample": "%d reduces in %.1f s on one thread" % (n, dt1)}}
    out = {}
    for name, parts_bits, got, dt, exact in checks:
        want = oracle.allreduce_threads(parts_bits, dt, cores)
        if exact:
            ok = oracle.same_result(got, want, dt)
        else:
            g, o = oracle.decode(got, dt), oracle.decode(want, dt)
            rtol = {oracle.F32: 1e-5, oracle.F16: 2e-3, oracle.BF16: 1.6e-2}[dt]
            with np.errstate(invalid="ignore"):
                ok = (np.isnan(g) & np.isnan(o)) | (np.abs(g - o) <= 1e-3 + rtol * np.abs(o))
        bad = int(np.count_nonzero(~ok))
        out[name] = {"elements": int(ok.size), "mismatches": bad, "rule": "bit-exact" if exact else "tolerance",
                     "ok": bad == 0}
        log("output check %s: %d of %d differ (%s)" % (name, bad, ok.size, "bit-exact" if exact else "tolerance"))
    return result, out


def run_sweep(comm_cls, args, stream):
    import torch
    import message_allreduce_amd as llar
    sizes = [1 << k for k in range(7, 27)]
    res = {"sizes": sizes, "protocols": {}}
    rows = {PROTO_NAMES[p]: [] for p in (1, 2, 3, 4, 5, 0)}
    comm = comm_cls(N_RANKS, torch.bfloat16, BIG_BYTES)
    try:
        for nbytes in sizes:
            n = nbytes // 2
            _, parts = device_inputs(5, N_RANKS, n, "normal", 1.0, rep=nbytes)
            out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
            steps = 200 if nbytes <= (1 << 20) else 20
            for proto in (1, 2, 3, 4, 5, 0):
                name = PROTO_NAMES[proto]
                if proto in (1, 2, 3) and nbytes > (8 << 20):
                    continue
                try:
                    us = time_calls(comm, parts, out, proto, steps, 10, stream)
                    dev_med, dev_min = device_side_us(comm, parts, out, proto, 40 if nbytes <= (1 << 20) else 10, stream)
                except llar.LlarError as e:
                    log("sweep %s %d: %s" % (name, nbytes, e))
                    continue
                gbps = (N_RANKS + 1) * nbytes / (us * 1e-6) / 1e9
                rows[name].append({"bytes": nbytes, "us_per_call": round(us, 3), "device_us": round(dev_med, 3),
                                   "device_us_min": round(dev_min, 3), "GBps": round(gbps, 1),
                                   "selected": PROTO_NAMES[comm.select_protocol(nbytes)] if proto == 0 else name})
                log("sweep %-18s %9d B  %8.2f us/call  %8.2f us device  %8.1f GB/s" % (name, nbytes, us, dev_med, gbps))
            del parts, out
        for name, rr in rows.items():
            if rr:
                a, b = fit_alpha_beta([r["bytes"] for r in rr], [r["us_per_call"] for r in rr])
                res["protocols"][name] = {"rows": rr, "alpha_us": a, "beta_us_per_byte": b}
    finally:
        comm.close()
    return res


def run_auto_sweep(comm, parts_big, stream):
    """The AUTO protocol at 128 B .. 64 MiB per rank (20 powers of two) on the
    N = 8 bf16 communicator: per-call microseconds of back-to-back calls
    (HIP events), the device-side span, effective GB/s over (N + 1) x S, and
    the alpha + beta * size fit over all sizes and over each protocol's
    sizes.  The inputs are the leading elements of the 64 MiB partials."""
    import torch
    sizes = [1 << k for k in range(7, 27)]
    rows = []
    for nbytes in sizes:
        n = nbytes // 2
        parts = [p[:n] for p in parts_big]
        out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        steps = 200 if nbytes <= (1 << 20) else 20
        us = time_calls(comm, parts, out, 0, steps, 10, stream)
        dev_med, dev_min = device_side_us(comm, parts, out, 0, 40 if nbytes <= (1 << 20) else 10, stream)
        gbps = (N_RANKS + 1) * nbytes / (us * 1e-6) / 1e9
        proto = PROTO_NAMES[comm.select_protocol(nbytes)]
        rows.append({"bytes": nbytes, "protocol": proto, "us_per_call": round(us, 3), "calls_timed": steps,
                     "device_us": round(dev_med, 3), "device_us_min": round(dev_min, 3), "GBps": round(gbps, 1)})
        log("sweep auto %9d B (%s): %8.2f us/call, %8.2f us device, %8.1f GB/s" % (nbytes, proto, us, dev_med, gbps))
        del parts, out
    a, b = fit_alpha_beta([r["bytes"] for r in rows], [r["us_per_call"] for r in rows])
    fits = {"all": {"alpha_us": round(a, 4), "beta_ps_per_byte": round(b * 1e6, 4), "sizes": len(rows)}}
    for proto in sorted({r["protocol"] for r in rows}):
        rr = [r for r in rows if r["protocol"] == proto]
        if len(rr) >= 2:
            a, b = fit_alpha_beta([r["bytes"] for r in rr], [r["us_per_call"] for r in rr])
            fits[proto] = {"alpha_us": round(a, 4), "beta_ps_per_byte": round(b * 1e6, 4), "sizes": len(rr)}
    log("sweep fit: %s" % json.dumps(fits))
    return {"workload": "allreduce, N=8 emulated ranks, bf16, AUTO, 128 B .. 64 MiB per rank",
            "rows": rows, "fit_T_eq_alpha_plus_beta_size": fits}


ATOMIC_KINDS = {"f32_all_xcds": 0, "f32_one_xcd": 4, "f32_all_xcds_one_window": 8,
                "f32_8way_cross_xcd": 16, "pk_bf16_all_xcds": 1, "pk_bf16_one_xcd": 5,
                "pk_bf16_8way_cross_xcd": 17, "pk_f16_all_xcds": 2}


def measure_atomic_ceiling():
    """Throughput of no-return device-scope float atomics issued with the
    LL128 producers' lane pattern (whole 128-byte lines per half wave), in G
    lane operations per second: binary32, packed bfloat16 and packed
    binary16; from all eight XCDs or one; private target lines, one window
    for all, or lines shared by eight workgroups on eight XCDs (the LL128
    pattern: the ranks of a slice add into the same lines)."""
    import message_allreduce_amd as llar
    res = {name: round(max(llar.llar_floor_measure(7, k) for _ in range(2)), 2) for name, k in ATOMIC_KINDS.items()}
    res["unit"] = "G lane operations per second"
    return res


def ll128_requests(n_ranks, n, chunk_elems, acc16):
    """Memory-side atomic requests one LL128 call issues: per rank and line,
    one for each 64-byte half of the line that holds data (the first half
    always does; the second once the line holds more than 15 binary32 or 31
    16-bit elements) and one for the count -- three per full line, which
    the TCC_ATOMIC counter confirms."""
    K = 63 if acc16 else 31
    half = 31 if acc16 else 15
    total = 0
    for c0 in range(0, n, chunk_elems):
        ln = min(chunk_elems, n - c0)
        full, rest = divmod(ln, K)
        total += full * 3 + ((3 if rest > half else 2) if rest else 0)
    return total * n_ranks


def ll128_lane_ops(n_ranks, n, chunk_elems, acc16):
    """Atomic lane operations one LL128 call issues: every rank adds each of
    its elements into its line (one binary32 add per element, or one packed
    16-bit pair per dword of a line, slot 0's dword included), and adds its
    count once per line it contributed to."""
    K = 63 if acc16 else 31
    total = 0
    for c0 in range(0, n, chunk_elems):
        ln = min(chunk_elems, n - c0)
        lines = -(-ln // K)
        if acc16:
            full, rest = divmod(ln, K)
            data = full * 32 + ((rest + 1 + 1) // 2 if rest else 0)
        else:
            data = ln
        total += data + lines
    return total * n_ranks


def to_bits(t):
    """Host copy of a bf16 device tensor as its bit patterns."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="calls in each timed region of the headline")
    ap.add_argument("--warmup", type=int, default=200, help="untimed calls before them")
    ap.add_argument("--big-steps", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing and the output check")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the send/recv, ReduceScatter, AllGather timings")
    ap.add_argument("--no-sweep", action="store_true", help="skip the AUTO size sweep")
    ap.add_argument("--sweep-all", action="store_true", help="also sweep every protocol")
    ap.add_argument("--sweep-out", default="sweep.json", help="where --sweep-all writes its rows and fits")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the N ranks are emulated inside a single MI355X "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import message_allreduce_amd as llar
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    checks = []  # (name, partial bits, GPU output bits, dtype code, bit-exact?)

    log("floor microbenchmarks")
    floor = measure_floor()
    log(json.dumps(floor))
    ceiling = measure_atomic_ceiling()
    log("atomic ceiling: %s" % json.dumps(ceiling))

    # ---- headline: 16 KiB bf16, N = 8, AUTO: exactly --steps calls per timed region
    n_small = SMALL_BYTES // 2
    bits_small, parts = device_inputs(5, N_RANKS, n_small, "normal", 1.0)
    out = torch.empty(n_small, dtype=torch.bfloat16, device="cuda")
    comm = llar.Communicator(N_RANKS, torch.bfloat16, BIG_BYTES)
    proto_small = comm.select_protocol(SMALL_BYTES)
    geo_small = comm.geometry(n_small, 0)
    log("16 KiB: protocol %s geometry %s" % (PROTO_NAMES[proto_small], geo_small))
    torch.cuda.synchronize()
    us = time_calls(comm, parts, out, 0, args.steps, args.warmup, stream)
    us_graph = time_graph(comm, parts, out, 0, args.steps, stream) if not args.no_graph else None
    per_graph, replays = graph_split(args.steps)
    # spread of the back-to-back rate over five more batches (not the headline)
    us_min, us_med, us_p90 = time_batches(comm, parts, out, 0, 5 * args.steps, 0, stream)
    dev_med, dev_min = device_side_us(comm, parts, out, 0, 60, stream)
    torch.cuda.synchronize()
    checks.append(("allreduce_16KiB_x8_bf16_auto", bits_small, to_bits(out), 2, True))
    log("16 KiB: %.3f us per call (%d back-to-back calls), %s us per call in graphs (%d calls), device-side "
        "median %.3f us (min %.3f)" % (us, args.steps, us_graph, args.steps, dev_med, dev_min))

    # ---- the same reduce behind a grid-wide barrier (what the flags replace)
    comm.set_option("barrier_ablation", 1)
    try:
        _, ab_us, _ = time_batches(comm, parts, out, 1, 5 * args.steps, args.warmup, stream)
        ab_dev_med, ab_dev_min = device_side_us(comm, parts, out, 1, 60, stream)
    finally:
        comm.set_option("barrier_ablation", 0)
    _, ll_us, _ = time_batches(comm, parts, out, 1, 5 * args.steps, 0, stream)
    ll_dev_med, _ = device_side_us(comm, parts, out, 1, 60, stream)
    log("16 KiB barrier ablation: %.3f us per call, device %.3f us; LL %.3f us per call, device %.3f us"
        % (ab_us, ab_dev_med, ll_us, ll_dev_med))

    # ---- 64 MiB bf16, N = 8, AUTO
    n_big = BIG_BYTES // 2
    bits_big, parts_big = device_inputs(5, N_RANKS, n_big, "normal", 1.0)
    out_big = torch.empty(n_big, dtype=torch.bfloat16, device="cuda")
    proto_big = comm.select_protocol(BIG_BYTES)
    geo_big = comm.geometry(n_big, 0)
    big_calls = max(50, args.big_steps)  # 5 batches of >= 10 back-to-back calls: the first launch's gap amortised
    us_big_min, us_big, us_big_p90 = time_batches(comm, parts_big, out_big, 0, big_calls, 5, stream)
    torch.cuda.synchronize()
    checks.append(("allreduce_64MiB_x8_bf16_auto", bits_big, to_bits(out_big), 2, True))
    alg_bytes = (N_RANKS + 1) * BIG_BYTES
    gbps = alg_bytes / (us_big * 1e-6) / 1e9
    log("64 MiB: protocol %s geometry %s: %.1f us, %.1f GB/s" % (PROTO_NAMES[proto_big], geo_big, us_big, gbps))
    copy_gbps = llar.llar_floor_measure(4, 1024)

    sweep = None
    if not args.no_sweep:
        log("AUTO size sweep")
        sweep = run_auto_sweep(comm, parts_big, stream)
    comm.close()
    del out_big

    traffic, traffic_src = profiled_traffic(os.path.join(ROOT, "message_allreduce_amd", "csrc", "llar_kernels.hip"),
                                            TRAFFIC_PROFILE)
    # value: the faster of the two ways a caller launches the reduce --
    # stream-ordered calls, or replay of a graph of captured calls (a
    # captured decode step); both timed regions hold exactly --steps calls
    graph_faster = us_graph is not None and us_graph < us
    value = us_graph if graph_faster else us
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(value / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: N(0,1) partials drawn from seed [5, 0], resident in HBM",
        "config": {"workload": "allreduce, N=8 emulated ranks x 16 KiB bf16 (8192 elements per rank), AUTO protocol",
                   "n_ranks": N_RANKS, "bytes_per_rank": SMALL_BYTES, "protocol": PROTO_NAMES[proto_small],
                   "geometry": geo_small,
                   "launch": ("hipGraph replay: %d captured calls per graph, %d replays" % (per_graph, replays)
                              if graph_faster else "stream-ordered back-to-back calls"),
                   "calls_timed": args.steps},
        "latency": dict(floor, **{"device_us_median": round(dev_med, 3), "device_us_min": round(dev_min, 3),
                                  "device_over_floor": round(dev_med / floor["floor_us"], 3),
                                  "device_over_rt_plus_store": round(dev_med / floor["floor_rt_plus_store_us"], 3),
                                  "per_call_over_floor_plus_launch": round(
                                      value / (floor["floor_us"] + floor["empty_launch_us"]), 3),
                                  "per_call_graph_over_floor_plus_graph_launch": None if us_graph is None else round(
                                      us_graph / (floor["floor_us"] + floor["empty_launch_graph_us"]), 3),
                                  "per_call_stream_us": round(us, 3),
                                  "per_call_graph_us": None if us_graph is None else round(us_graph, 3),
                                  "timed_calls": {"stream": args.steps, "graph": 0 if us_graph is None else args.steps,
                                                  "graph_calls_per_graph": per_graph},
                                  "per_call_stream_batches_us": {"batches": 5, "calls_per_batch": args.steps,
                                                                 "min": round(us_min, 3), "median": round(us_med, 3),
                                                                 "p90": round(us_p90, 3)},
                                  "device_calls_timed": 60}),
        "barrier_ablation": {"workload": "the same 16 KiB x 8 one-shot reduce, grid-wide barrier instead of LL flags",
                             "per_call_us": round(ab_us, 3), "device_us_median": round(ab_dev_med, 3),
                             "device_us_min": round(ab_dev_min, 3), "ll_per_call_us": round(ll_us, 3),
                             "ll_device_us_median": round(ll_dev_med, 3),
                             "barrier_cost_device_us": round(ab_dev_med - ll_dev_med, 3)},
        "bandwidth_64MiB": {"protocol": PROTO_NAMES[proto_big], "geometry": geo_big,
                            "us": {"min": round(us_big_min, 2), "median": round(us_big, 2), "p90": round(us_big_p90, 2)},
                            "calls_timed": {"batches": 5, "calls_per_batch": big_calls // 5},
                            "GBps": round(gbps, 1), "algorithmic_bytes": alg_bytes,
                            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                            "copy_GBps_measured": round(copy_gbps, 1),
                            "traffic_source": traffic_src},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "kernel": "%s, 64 MiB x 8 bf16" % PROTO_NAMES[proto_big]},
        "atomic_ceiling": ceiling,
    }
    if sweep is not None:
        result["sweep"] = sweep
    if not args.no_rows:
        log("other collectives")
        result["rows"] = measure_rows(stream, min(args.steps, 1000))
        result["rows"]["device_api_fused_epilogue"] = measure_device_api(stream, min(args.steps, 1000))
        log("fixed workloads")
        result["workloads"] = measure_workloads(stream, min(args.steps, 1000), floor["floor_us"], ceiling, checks)
    if not args.no_cpu:
        log("cpu baseline (oracle) and output check")
        result["cpu_baseline"], result["output_check"] = cpu_baseline(args.cpu_seconds, checks)
    if args.sweep_all:
        log("sweep of every protocol")
        sw = run_sweep(llar.Communicator, args, stream)
        if os.path.dirname(args.sweep_out):
            os.makedirs(os.path.dirname(args.sweep_out), exist_ok=True)
        with open(args.sweep_out, "w") as f:
            json.dump(sw, f, indent=1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
