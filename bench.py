#!/usr/bin/env python3
"""Benchmark: one step of the INT8-compressed gradient AllReduce compute on
one MI355X, for W simulated data-parallel ranks.

A step is the whole per-device hot path on one batch of gradients already
resident in HBM:
  1. quantize every rank's gradient (load + unscale, per-unit absmax, scale,
     int8 codes): gq_quantize with fused maxima, all W ranks in one call;
  2. reduce the W ranks' dequantized codes in fp32 in rank order and
     requantize the sum: gq_reduce_requantize (the sum stays on chip).
The chunk plans and unit tables are built once at set-up (they depend only
on the tensor shapes).

Prints one JSON line.  The default workload is the largest one: W = 16
ranks, each holding one fp32 gradient of 2^28 elements (1 GiB) with
Student-t(3) values, one scale per 128 KiB chunk (8,192 chunks); --workload
picks another of the five synthetic workloads.

Every run also checks what it timed: the outputs of the last timed step
(every rank's scales and codes, the requantized scales and codes) and the
fp32 rank-order sum of one more reduce are compared with the CPU oracle on
every element, unit range by unit range, on the same host inputs; that
oracle pass is timed on one host core and reported as the CPU baseline.  A
mismatch makes the run exit with status 4.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
METRIC = "GB/s gradient input quantized+reduced on 1 MI355X; % of HBM peak"
KERNEL_SRC = os.path.join(ROOT, "gradient_compression_allreduce_amd", "csrc", "gq_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source
    (else None)."""
    path = os.path.join(PROFILES, "traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return int(kv["traffic_bytes_per_launch"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def unit_offsets(w, plan):
    if w.units == "tensor":
        return w.toff.copy()
    parts = [np.zeros(1, dtype=np.int64)]
    for t, size in enumerate(w.sizes):
        parts.append(plan(int(size), w.elem_bytes)[1:] + w.toff[t])
    return np.concatenate(parts)


def bucket_bounds(w, plan, bucket_bytes=None):
    """Unit indices where the gradient buckets start (greedy buckets of
    whole tensors of bucket_bytes if given, else the workload's own
    buckets, else 25 MiB), plus the end."""
    if w.buckets and bucket_bytes is None:
        groups = w.buckets
    else:
        bucket_bytes = bucket_bytes or 25 * 1024 * 1024
        groups, start, acc = [], 0, 0
        for t, size in enumerate(w.sizes):
            b = int(size) * w.elem_bytes
            if acc > 0 and acc + b > bucket_bytes:
                groups.append((start, t))
                start, acc = t, 0
            acc += b
        groups.append((start, len(w.sizes)))
    if w.units == "tensor":
        first_unit = np.arange(len(w.sizes) + 1)
    else:
        counts = [len(plan(int(size), w.elem_bytes)) - 1 for size in w.sizes]
        first_unit = np.concatenate([[0], np.cumsum(counts)])
    return np.array([first_unit[a] for a, _ in groups] + [first_unit[-1]], dtype=np.int64)


def algorithmic_bytes(W, n, e, U):
    """Bytes the method must move with one read of every input:
    quantize: W*n*e in + W*n codes out + W*U scales out;
    reduce+requantize: W*n codes in + W*U scales in + n codes out + U scales out."""
    bq = W * n * (e + 1) + 4 * W * U
    br = n * (W + 1) + 4 * W * U + 4 * U
    return bq, br


def stage_kernels(gq, units, kind, in_mul):
    """Names of the kernels that run the two stages on a table (the form
    each stage takes decides which)."""
    dt = gq.GQ_F32 if kind == 0 else gq.GQ_F16
    plan = gq.gq_units_launch_plan(units, dt, in_mul)
    if plan["q_form"] == gq.GQ_FORM_SHORT_UNITS:
        qkernel = "k_quantize_small"
    elif plan["q_form"] == gq.GQ_FORM_TWO_PASS:
        qkernel = "k_tile_absmax+k_quantize"
    else:
        qkernel = ("k_quantize_chunk" if gq.gq_units_schedule(units, dt) == gq.GQ_SCHED_CHUNK
                   else "k_quantize_layer")
    if plan["r_form"] == gq.GQ_FORM_SHORT_UNITS:
        rkernel = "k_reduce_pieces"
    elif plan["r_form"] == gq.GQ_FORM_TWO_PASS:
        rkernel = "k_reduce"
    else:
        # wide (16384-element) and chunk-wide (32768) tiles: one kernel
        # template on 512 and 1024 threads
        rkernel = "k_reduce_coop" if gq.gq_units_reduce_tile(units) == 8192 else "k_reduce_coop_wide"
    return qkernel, rkernel


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def unit_batches(off, min_elems):
    """Consecutive unit ranges [ua, ub) of at least min_elems elements each
    (the last one may be shorter).  Units are independent, so the oracle's
    result on a range of whole units is its result on the whole workload,
    restricted to that range."""
    U = off.size - 1
    out, ua = [], 0
    while ua < U:
        ub = int(np.searchsorted(off, off[ua] + min_elems, side="left"))
        ub = min(max(ub, ua + 1), U)
        out.append((ua, ub))
        ua = ub
    return out


def f32_mismatches(a, b):
    """Elements of two float32 arrays that differ bitwise (NaNs compared by
    NaN-ness only)."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    bad = (na != nb) | (~na & ~nb & (a.view(np.uint32) != b.view(np.uint32)))
    return int(np.count_nonzero(bad))


def input_checksums(w, xs):
    """64-bit FNV-1a of every rank's host input buffer (hex), taken in
    parallel host threads (the C checksum releases the interpreter)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=max(1, min(16, len(xs)))) as ex:
        return ["%016x" % c for c in ex.map(w.checksum, xs)]


def oracle_check(w, xs, off, kind, got, min_seconds=10.0, max_reps=20, batch_elems=1 << 23):
    """Run the oracle (single-threaded C, as it stands) on the same host
    inputs, unit range by unit range, one host thread pinned to one core,
    and compare its outputs with the GPU's on every element.

    got: host-side access to the GPU outputs: got["scale"][w] (numpy, all
    units), got["scale_out"] (numpy), and callables got["codes"](w, a, b),
    got["r"](a, b), got["q_out"](a, b) returning element ranges.

    The comparing pass is timed (oracle calls only); if it took less than
    min_seconds, whole oracle passes are repeated (not compared) until
    that much CPU work has been timed, and the median is reported."""
    from oracle import Oracle
    o = Oracle()
    batches = unit_batches(off, batch_elems)
    bad = {"codes": 0, "scales": 0, "r": 0, "scale_out": 0, "q_out": 0}
    first_bad = None
    old_aff = os.sched_getaffinity(0)
    core = min(old_aff)
    os.sched_setaffinity(0, {core})
    try:
        def one_pass(compare):
            nonlocal first_bad
            t_sum = 0.0
            for ua, ub in batches:
                a, b = int(off[ua]), int(off[ub])
                loc = off[ua:ub + 1] - a
                sl = [x[a:b] for x in xs]
                t0 = time.perf_counter()
                want = o.allreduce_step(sl, kind, loc, w.in_mul)
                t_sum += time.perf_counter() - t0
                if not compare:
                    continue
                before = sum(bad.values())
                for r in range(w.W):
                    bad["scales"] += f32_mismatches(got["scale"][r][ua:ub], want["scale"][r])
                    bad["codes"] += int(np.count_nonzero(got["codes"](r, a, b) != want["q"][r]))
                bad["r"] += f32_mismatches(got["r"](a, b), want["r"])
                bad["scale_out"] += f32_mismatches(got["scale_out"][ua:ub], want["scale_out"])
                bad["q_out"] += int(np.count_nonzero(got["q_out"](a, b) != want["q_out"]))
                if first_bad is None and sum(bad.values()) > before:
                    first_bad = {"units": [ua, ub], "elements": [a, b]}
            return t_sum

        times = [one_pass(True)]
        while sum(times) < min_seconds and len(times) < max_reps:
            times.append(one_pass(False))
    finally:
        os.sched_setaffinity(0, old_aff)
    U = off.size - 1
    compared = {"codes": w.W * w.n, "scales": w.W * U, "r": w.n, "scale_out": U, "q_out": w.n}
    parity = {"bit_exact": sum(bad.values()) == 0,
              "elements_compared": int(sum(compared.values())),
              "compared": compared, "mismatches": bad, "first_mismatch": first_bad,
              "rule": "bitwise; NaN compared by NaN-ness",
              "unit_batches": len(batches)}
    dt = float(np.median(times))
    nbytes = w.W * w.n * w.elem_bytes
    base = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds_per_step": dt, "repetitions": len(times),
            "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model(),
            "sample": "the whole workload (%d ranks x %d elements, every unit), in %d unit "
                      "ranges: quantize, rank-order reduce and requantize; %d pass(es), "
                      "median; the first pass's outputs are the parity check; one host "
                      "thread pinned to core %d" % (w.W, w.n, len(batches), len(times), core)}
    return parity, base


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle pass (and with it the parity check of the timed "
                         "step): for profiling runs only")
    ap.add_argument("--pipeline", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the two-stream bucket pipeline (outside the step)")
    ap.add_argument("--bucket-mib", type=float, default=None,
                    help="pipeline bucket size (default: the workload's buckets, else 25)")
    ap.add_argument("--adaptive", action="store_true",
                    help="per-chunk workloads: feed the adaptive chunker with steps timed "
                         "at chunk sizes of 32 KiB .. 1 MiB and report its choice")
    ap.add_argument("--no-ab", action="store_true",
                    help="skip the quantization-off comparison (fp32 sum + error report)")
    ap.add_argument("--graph-reps", type=int, default=None,
                    help="also time the step replayed from a HIP graph of this many "
                         "repetitions (default: 100 for the launch-bound 1M-element "
                         "workload, else off)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the simulated ranks all live in one device's "
              "memory and the library has no multi-GPU exchange; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(2)
    from datagen import get_workload
    from gradient_compression_allreduce_amd import gq

    w = get_workload(args.workload, seed=args.seed)
    if args.graph_reps is None:
        args.graph_reps = 100 if args.workload == 1 else 0
    kind = 0 if w.kind == "f32" else 1
    off = unit_offsets(w, gq.gq_plan_chunks)
    U = off.size - 1
    # §2.1 chunk plan of every communication buffer (buckets, else tensors)
    groups = w.buckets if w.buckets else [(t, t + 1) for t in range(len(w.sizes))]
    n_chunks = 0
    for a, b in groups:
        nb = int(w.toff[b] - w.toff[a])
        n_chunks += len(gq.gq_plan_chunks(nb, w.elem_bytes)) - 1

    log("workload", w.name, "W", w.W, "n", w.n, "units", U, "chunks", n_chunks)
    t0 = time.perf_counter()
    xs = []
    for r in range(w.W):
        xs.append(w.fill(r))
        if w.n >= (1 << 26):
            log("  rank %d generated" % r)
    log("generated inputs in %.1f s" % (time.perf_counter() - t0))
    t0 = time.perf_counter()
    checksums = input_checksums(w, xs)
    log("input checksums in %.1f s" % (time.perf_counter() - t0))
    dev = torch.device("cuda")
    tdt = torch.float32 if kind == 0 else torch.float16
    dx = []
    for x in xs:
        src = torch.from_numpy(x.view(np.float16) if kind == 1 else x)
        dx.append(src.to(dev))
    units = gq.gq_units_create(off)
    scales = [torch.empty(U, dtype=torch.float32, device=dev) for _ in range(w.W)]
    codes = [torch.empty(w.n, dtype=torch.int8, device=dev) for _ in range(w.W)]
    s_out = torch.empty(U, dtype=torch.float32, device=dev)
    q_out = torch.empty(w.n, dtype=torch.int8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        gq.gq_quantize(dx, units, scales, codes, in_mul=w.in_mul, stream=stream)
        gq.gq_reduce_requantize(codes, scales, units, s_out, q_out, stream=stream)

    # practical ceiling: a plain device-to-device copy of the same volume
    bq, br = algorithmic_bytes(w.W, w.n, w.elem_bytes, U)
    cp_src = torch.empty(int(bq // 2), dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    for _ in range(2):
        cp_dst.copy_(cp_src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        cp_dst.copy_(cp_src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * cp_src.numel() * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del cp_src, cp_dst

    pipeline = None
    if args.pipeline:
        # the two-stream bucket pipeline (two code slots per rank), in both
        # modes, same inputs, same requantized result
        bounds = bucket_bounds(w, gq.gq_plan_chunks,
                               int(args.bucket_mib * 1024 * 1024) if args.bucket_mib else None)
        pipeline = []
        if bounds.size - 1 < 2:
            # one tensor larger than a bucket is a bucket of its own: nothing
            # to pipeline
            pipeline = {"skipped": "one bucket (a tensor larger than the bucket size is a "
                                   "bucket of its own)"}
        for mode, name in (((gq.GQ_PIPE_OVERLAP, "overlap"), (gq.GQ_PIPE_SERIAL, "serial"))
                           if bounds.size - 1 >= 2 else ()):
            pipe = gq.gq_pipe_create(off, bounds, mode)
            se, su = gq.gq_pipe_slots(pipe)
            q_slots = [torch.empty(se, dtype=torch.int8, device=dev) for _ in range(2 * w.W)]
            s_slots = [torch.empty(su, dtype=torch.float32, device=dev) for _ in range(2 * w.W)]
            p_s_out = torch.empty(U, dtype=torch.float32, device=dev)
            p_q_out = torch.empty(w.n, dtype=torch.int8, device=dev)

            def pstep():
                gq.gq_pipe_step(pipe, dx, q_slots, s_slots, p_s_out, p_q_out, in_mul=w.in_mul,
                                stream=stream)

            for _ in range(args.warmup):
                pstep()
            torch.cuda.synchronize()
            p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            p0.record(stream)
            for _ in range(args.steps):
                pstep()
            p1.record(stream)
            torch.cuda.synchronize()
            if gq.gq_pipe_faults(pipe):
                print("a bounded cross-group wait gave up in the pipeline: results invalid",
                      file=sys.stderr)
                sys.exit(3)
            step()
            torch.cuda.synchronize()
            same = bool(torch.equal(p_q_out, q_out)) and bool(
                torch.equal(p_s_out.view(torch.int32), s_out.view(torch.int32)))
            p_ms = p0.elapsed_time(p1) / args.steps
            sched = gq.gq_pipe_schedule(pipe, kind, w.in_mul)
            pipeline.append({"mode": name, "buckets": int(bounds.size - 1),
                             "schedule": {gq.GQ_PIPE_SCHED_ALTERNATE: "alternate",
                                          gq.GQ_PIPE_SCHED_EVENTS: "events",
                                          gq.GQ_PIPE_SCHED_SERIAL: "serial"}[sched],
                             "ms_per_step": round(p_ms, 4),
                             "value": round(w.W * w.n * w.elem_bytes / (p_ms * 1e-3) / 1e9, 2),
                             "code_slot_bytes_per_rank": int(2 * se),
                             "same_result_as_step": same})
            del pipe, q_slots, s_slots, p_s_out, p_q_out

    adaptive = None
    if args.adaptive and w.units == "chunk":
        # the adaptive chunker fed with measured steps at several chunk
        # sizes (each size is its own plan: other chunks, other scales)
        ch = gq.gq_chunker_create()
        cands = []
        for kib in (32, 64, 128, 256, 512, 1024):
            cb = kib * 1024
            parts = [np.zeros(1, dtype=np.int64)]
            for t, size in enumerate(w.sizes):
                parts.append(gq.gq_plan_chunks(int(size), w.elem_bytes, cb)[1:] + w.toff[t])
            off_c = np.concatenate(parts)
            units_c = gq.gq_units_create(off_c)
            Uc = off_c.size - 1
            sc_c = [torch.empty(Uc, dtype=torch.float32, device=dev) for _ in range(w.W)]
            so_c = torch.empty(Uc, dtype=torch.float32, device=dev)

            def cstep():
                gq.gq_quantize(dx, units_c, sc_c, codes, in_mul=w.in_mul, stream=stream)
                gq.gq_reduce_requantize(codes, sc_c, units_c, so_c, q_out, stream=stream)

            for _ in range(2):
                cstep()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            for _ in range(5):
                cstep()
            c1.record(stream)
            torch.cuda.synchronize()
            if gq.gq_units_faults(units_c):
                print("a bounded cross-group wait gave up: results invalid", file=sys.stderr)
                sys.exit(3)
            c_ms = c0.elapsed_time(c1) / 5
            gq.gq_chunker_update(ch, cb, c_ms * 1e-3 / Uc)   # seconds per chunk
            cands.append({"chunk_bytes": cb, "chunks": int(Uc), "ms_per_step": round(c_ms, 4)})
            del units_c, sc_c, so_c
        pred = gq.gq_chunker_predict(ch)
        adaptive = {"candidates": cands, "predicted_chunk_bytes": pred,
                    "ms_at_prediction": next(c["ms_per_step"] for c in cands
                                             if c["chunk_bytes"] == pred),
                    "ms_at_128KiB": next(c["ms_per_step"] for c in cands
                                         if c["chunk_bytes"] == 131072)}

    ab = None
    if not args.no_ab:
        # the precision check with quantization switched off, outside the
        # timed step: the fp32 rank-order sum of the same gradients and the
        # per-unit error report of the INT8 result against it
        ref = torch.empty(w.n, dtype=torch.float32, device=dev)
        stats = torch.empty(U * gq.GQ_STATS, dtype=torch.float64, device=dev)
        step()
        gq.gq_sum_f32(dx, ref, in_mul=w.in_mul, stream=stream)
        gq.gq_error_report(q_out, s_out, ref, units, stats, stream=stream)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        for _ in range(5):
            gq.gq_sum_f32(dx, ref, in_mul=w.in_mul, stream=stream)
        e[1].record(stream)
        for _ in range(5):
            gq.gq_error_report(q_out, s_out, ref, units, stats, stream=stream)
        e[2].record(stream)
        torch.cuda.synchronize()
        sum_ms = e[0].elapsed_time(e[1]) / 5
        rep_ms = e[1].elapsed_time(e[2]) / 5
        st = stats.cpu().numpy().reshape(U, gq.GQ_STATS)
        col = {k: i for i, k in enumerate(gq.STATS)}
        fin = np.isfinite(st[:, col["cos"]])
        ab = {"fp32_sum_ms": round(sum_ms, 4),
              "fp32_sum_GBps": round((w.W * w.n * w.elem_bytes + 4 * w.n) / (sum_ms * 1e-3) / 1e9, 1),
              "report_ms": round(rep_ms, 4),
              "report_GBps": round(5 * w.n / (rep_ms * 1e-3) / 1e9, 1),
              "units_non_finite": int((~fin).sum()),
              "worst_max_rel_err": float(np.max(st[fin, col["max_rel_err"]])) if fin.any() else None,
              "mean_mean_rel_err": float(np.mean(st[fin, col["mean_rel_err"]])) if fin.any() else None,
              "min_cos": float(np.min(st[fin, col["cos"]])) if fin.any() else None}
        del ref, stats

    graph = None
    if args.graph_reps > 0:
        # the same step, captured once into a HIP graph of graph_reps
        # repetitions (launch-bound workloads); no allocation or memset is
        # recorded: the library's compute calls make none
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for _ in range(args.graph_reps):
                    gq.gq_quantize(dx, units, scales, codes, in_mul=w.in_mul, stream=cap)
                    gq.gq_reduce_requantize(codes, scales, units, s_out, q_out, stream=cap)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph = {"reps": args.graph_reps,
                 "ms_per_step": round(g0.elapsed_time(g1) / args.graph_reps, 4)}
        del g

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the stage breakdown and the kernels' durations (the roofline): K steps
    # with an event before each launch and one after the last, on the
    # kernels' own stream, right before the timed region
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        ev[2 * k].record(stream)
        gq.gq_quantize(dx, units, scales, codes, in_mul=w.in_mul, stream=stream)
        ev[2 * k + 1].record(stream)
        gq.gq_reduce_requantize(codes, scales, units, s_out, q_out, stream=stream)
    ev[2 * args.steps].record(stream)
    torch.cuda.synchronize()
    q_ms = float(np.mean([ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(args.steps)]))
    r_ms = float(np.mean([ev[2 * k + 1].elapsed_time(ev[2 * k + 2]) for k in range(args.steps)]))
    step_ms = [ev[2 * k].elapsed_time(ev[2 * k + 2]) for k in range(args.steps)]
    instrumented_ms = ev[0].elapsed_time(ev[2 * args.steps]) / args.steps

    # the timed region: exactly K steps between two events, with nothing else
    # on the stream (an event recorded between two launches delays the
    # second by a few microseconds)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms = total_ms / args.steps
    faults = gq.gq_units_faults(units)
    if faults:
        print("a bounded cross-group wait gave up %d times: results invalid" % faults,
              file=sys.stderr)
        sys.exit(3)

    # what the last timed step left: every rank's scales and codes and the
    # requantized output.  One more reduce also writes the fp32 sum; its
    # requantized output must equal the timed step's.
    r_sum = None
    same_again = None
    if not args.no_cpu_baseline:
        keep_q, keep_s = q_out.clone(), s_out.clone()
        r_sum = torch.empty(w.n, dtype=torch.float32, device=dev)
        gq.gq_reduce_requantize(codes, scales, units, s_out, q_out, r_out=r_sum, stream=stream)
        torch.cuda.synchronize()
        same_again = bool(torch.equal(keep_q, q_out)) and bool(
            torch.equal(keep_s.view(torch.int32), s_out.view(torch.int32)))
        del keep_q, keep_s
        if gq.gq_units_faults(units):
            print("a bounded cross-group wait gave up: results invalid", file=sys.stderr)
            sys.exit(3)

    input_bytes = w.W * w.n * w.elem_bytes
    value = input_bytes / (ms * 1e-3) / 1e9
    b_alg = bq + br
    q_achieved = bq / (q_ms * 1e-3) / 1e9
    qkernel, rkernel = stage_kernels(gq, units, kind, w.in_mul)
    r_achieved = br / (r_ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.kind,
        "data": "synthetic",
        "config": {"workload": w.name, "W": w.W, "elements_per_rank": w.n,
                   "tensors": int(len(w.sizes)), "scale_units": U,
                   "scale_unit": w.units, "chunks": n_chunks,
                   "buckets": len(w.buckets) if w.buckets else None,
                   "seed": args.seed},
        "hbm_fraction": round(b_alg / (ms * 1e-3) / HBM_PEAK, 4),
        # bytes a rank would exchange (int8 codes + fp32 scales) over the
        # bytes of its fp32 gradient: the compression of the INT8 AllReduce
        "wire_bytes_vs_fp32": round((w.n + 4 * U) / (4.0 * w.n), 5),
        "algorithmic_bytes_per_step": b_alg,
        # per-step and per-stage times from K more steps with an event
        # around every launch (the events add a few microseconds per step)
        "instrumented_ms_per_step": round(instrumented_ms, 4),
        "step_ms_median": round(float(np.median(step_ms)), 4),
        "step_ms_min": round(float(np.min(step_ms)), 4),
        "stages_ms": {"quantize": round(q_ms, 4), "reduce_requantize": round(r_ms, 4)},
        "graph": graph,
        "pipeline": pipeline,
        "adaptive_chunk": adaptive,
        "ab_fp32": ab,
        # the quantize stage's kernel (one persistent launch on the per-chunk
        # and per-layer workloads), timed by the events around its launches
        "roofline": {"bound": "hbm", "kernel": qkernel,
                     "achieved": round(q_achieved, 1), "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": round(q_achieved / (HBM_PEAK / 1e9), 4),
                     "traffic": measured_traffic(qkernel, w.name),
                     "algorithmic_bytes_per_launch": bq},
        # the other stage's kernel, the same way
        "roofline_reduce": {"bound": "hbm", "kernel": rkernel,
                            "achieved": round(r_achieved, 1), "peak": HBM_PEAK / 1e9,
                            "unit": "GB/s", "frac": round(r_achieved / (HBM_PEAK / 1e9), 4),
                            "traffic": measured_traffic(rkernel, w.name),
                            "algorithmic_bytes_per_launch": br},
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "kernel_source": kernel_source_hash(),
        "wall_s": round(wall, 3),
        "input_checksums": {"fnv1a64": checksums},
        "parity": None,
    }
    ok = True
    if not args.no_cpu_baseline:
        log("CPU oracle on the same inputs: every element of the timed step ...")
        t0 = time.perf_counter()
        got = {"scale": [t.cpu().numpy() for t in scales],
               "scale_out": s_out.cpu().numpy(),
               "codes": lambda r, a, b: codes[r][a:b].cpu().numpy(),
               "r": lambda a, b: r_sum[a:b].cpu().numpy(),
               "q_out": lambda a, b: q_out[a:b].cpu().numpy()}
        parity, base = oracle_check(w, xs, off, kind, got)
        parity["requantized_again_with_sum_identical"] = same_again
        parity["seconds"] = round(time.perf_counter() - t0, 1)
        base["value"] = round(base["value"], 4)
        base["seconds_per_step"] = round(base["seconds_per_step"], 3)
        rec["parity"] = parity
        rec["cpu_baseline"] = base
        ok = parity["bit_exact"] and same_again
        log("parity:", "bit-exact" if ok else "MISMATCH", parity["mismatches"])
    print(json.dumps(rec), flush=True)
    if not ok:
        sys.exit(4)


if __name__ == "__main__":
    main()
