#!/usr/bin/env python3
"""Benchmark: bucketed gradient synchronisation on one MI355X.

Metric: effective HBM GB/s of one synchronisation, (N*P*b_in + P*b_out) /
t_sync, and its fraction of the 8 TB/s HBM peak.  A step is one whole
synchronisation of the workload: every bucket of the plan reduced over the N
virtual ranks in the fixed order, scaled by 1/N and written -- one launch of
ddp_sync_allreduce_avg.  Gradients sit in their bucket buffers (the
gradient-as-bucket-view layout), so flatten and unflatten are not needed in
the step; the same run also times the copy layout (flatten every rank, sync,
unflatten) and reports it under "copy_path".

Prints ONE JSON line.  Only one GPU is used: --gpus above 1 exits with 2.
Besides the metric and its roofline, the line carries (each can be skipped
with its --no-... flag):
  other_orders   the other summation order
  per_bucket     the same sync as one launch per bucket (loop and graph)
  cold_mall      the sync with the MALL flushed before each one
  ceiling        a probe of the reduce's bare access pattern
  cpu_baseline   the CPU oracle (one thread, and SEQ on all host cores)
  copy_path      flatten + sync + unflatten (eager and graph-replayed), and
                 the same step as one kernel over per-parameter tensors
  fused_sgd      the average fused into a momentum-SGD step (flat and
                 per-parameter tensors)
  overlap        syncs beside compute on a second stream
  rank_sweep_GBps, in_place, no_sync, env

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--workload resnet50|gpt1p3b|gpt1p3b_two_bucket|many_small|llama7b|tiny]
                       [--order ring|seq] [--cpu-seconds S] [--no-<section> ...]
       python bench.py --calibrate   (the plain-copy run that scales the HBM counters)
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "effective HBM GB/s (N·P·bytes read + P written) and % of peak per sync"
CSRC = os.path.join(ROOT, "gradient_allreduce_averaging_amd", "csrc")
# the library's device and launch code: every kernel source and header but the
# benchmark's own probe
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                        if f.endswith((".hip", ".h")) and f != "probe.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha():
    """sha256[:16] of the kernel sources (in name order) with comments and
    blank lines removed and each line stripped, so that only a change of code
    invalidates the counter data taken on it."""
    code = []
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        lines = (re.sub(r"//.*", "", line).strip() for line in text.splitlines())
        code.append(os.path.basename(path) + "\n" + "\n".join(line for line in lines if line))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def measured_traffic(workload, order, algorithmic_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they were taken on another version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    rec = table.get(f"{workload}/{order}")
    if not rec or rec.get("kernel_source_sha") != kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def side_by_side_streams(torch, tries=32):
    """Two streams whose kernels run side by side, and the number of streams
    tried.  HIP binds every stream to one of a few hardware queues
    (GPU_MAX_HW_QUEUES, 4 by default), and two streams bound to one queue run
    in submission order: a cross-stream wait in that queue holds back
    everything queued behind it, so a compute stream and an update stream
    that share a queue cannot overlap at all.  Checked by spinning a kernel
    on the first stream and seeing a tiny kernel on the second finish before
    it; torch hands out its pooled streams in turn, so the next candidate is
    another stream."""
    first = torch.cuda.Stream()
    x = torch.zeros(1, device="cuda:0")
    for k in range(1, tries + 1):
        second = torch.cuda.Stream()
        torch.cuda.synchronize()
        spun, tiny = torch.cuda.Event(), torch.cuda.Event()
        with torch.cuda.stream(first):
            torch.cuda._sleep(20_000_000)      # a bounded spin (clock cycles)
            spun.record(first)
        with torch.cuda.stream(second):
            x.add_(1.0)
            tiny.record(second)
        while True:
            t_done, s_done = tiny.query(), spun.query()
            if t_done or s_done:
                break
        torch.cuda.synchronize()
        if t_done and not s_done:
            return first, second, k
    return first, second, None


def run_environment(torch):
    """ROCm release, HIP runtime and the device's peak clocks, for the record."""
    env = {"hip_runtime": torch.version.hip, "torch": torch.__version__,
           "launch": "direct launches (no graph) in the timed loop"}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch has already loaded
        # hipDeviceAttributeClockRate = 5 and ...MemoryClockRate = 60 (both kHz),
        # ...MemoryBusWidth = 59 (bits), as numbered in ROCm 7's hip_runtime_api.h
        for key, attr, div in (("sclk_peak_mhz", 5, 1000), ("mclk_peak_mhz", 60, 1000),
                               ("mem_bus_bits", 59, 1)):
            v = ctypes.c_int(0)
            if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) == 0:
                env[key] = v.value // div
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    env["arch"] = getattr(props, "gcnArchName", "")
    env["compute_units"] = props.multi_processor_count
    return env


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="resnet50")
    ap.add_argument("--order", default="ring", choices=["ring", "seq"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-path", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-fused-sgd", action="store_true")
    ap.add_argument("--no-overlap", action="store_true")
    ap.add_argument("--no-no-sync", action="store_true")
    ap.add_argument("--no-in-place", action="store_true")
    ap.add_argument("--no-rank-sweep", action="store_true")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--no-per-bucket", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 10 times (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the N virtual ranks of a synchronisation live in that GPU's HBM", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gradient_allreduce_averaging_amd as ddp
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.calibrate:
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": a.numel() * 4, "copies": 10}), flush=True)
        return
    wl = W.workload(args.workload)
    order = args.order
    N = wl.n_ranks
    if wl.two_bucket:
        plan = ddp.plan_two_bucket(wl.numel, wl.regions, wl.dtype)
    else:
        plan = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, wl.dtype)
    P = plan.total
    tin = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    tout = torch.float32 if wl.out_dtype == "f32" else torch.bfloat16
    log(f"workload {wl.name}: N={N} P={P} buckets={plan.n_buckets} order={order} "
        f"{wl.dtype}->{wl.out_dtype}")

    flats = []
    for r in range(N):
        t = torch.empty(P, dtype=tin, device=dev)
        W.device_normal_(t, r, wl.stream, wl.sigma)
        flats.append(t)
    out = torch.empty(P, dtype=tout, device=dev)
    plan.prepare()
    stream = torch.cuda.current_stream()
    sync_bytes = wl.sync_bytes()

    prepared = {o: ddp.make_sync(plan, flats, out, o, stream=stream) for o in ("seq", "ring")}

    def sync(o=order):
        prepared[o]()

    # ---------------------------------------------------------------- timed
    # K back-to-back steps, wall clock between two synchronisations; one event
    # pair brackets the loop on the launch stream.
    for _ in range(args.warmup):
        sync()
    loop_a, loop_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop_a.record(stream)
    for _ in range(args.steps):
        sync()
    loop_b.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    gpu_ms_per_step = loop_a.elapsed_time(loop_b) / args.steps
    value = sync_bytes / (ms_per_step * 1e-3) / 1e9

    # The reduce kernel's average launch duration: the event pair around the
    # timed loop on the launch stream, over K back-to-back launches (one
    # kernel per step, so this is the kernel plus the launch gap).
    kern_ms = gpu_ms_per_step
    achieved = sync_bytes / (kern_ms * 1e-3) / 1e9
    # Spread: the same K steps again, each launch bracketed by its own event
    # pair (these add the event overhead of a few microseconds to each).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for a, b in ev:
        a.record(stream)
        sync()
        b.record(stream)
    torch.cuda.synchronize()
    launch_ms = [a.elapsed_time(b) for a, b in ev]
    log(f"sync: {ms_per_step * 1e3:.1f} us/step wall, {gpu_ms_per_step * 1e3:.1f} us/step on the "
        f"stream ({achieved:.0f} GB/s); single launches between events: median "
        f"{np.median(launch_ms) * 1e3:.1f} us, min {min(launch_ms) * 1e3:.1f} us")

    # ---------------------------------------------------------------- one launch per bucket
    # The same sync as DDP issues it, one all-reduce call per bucket
    # (ddp_bucket_allreduce_avg on each bucket's sub-ranges): driven from
    # Python, and replayed from a HIP graph that captured those launches.
    # Against the one-launch sync this is the launch overhead it saves.
    per_bucket = None
    if not args.no_per_bucket and 1 < plan.n_buckets <= 4096 and P < 10 ** 9:
        spans = [plan.bucket(b)[:2] for b in range(plan.n_buckets)]
        ins_b = [[f[base:base + ln] for f in flats] for ln, base in spans]
        outs_b = [out[base:base + ln] for ln, base in spans]
        side = torch.cuda.Stream()

        def per_bucket_sync():
            for xs_b, o_b in zip(ins_b, outs_b):
                ddp.bucket_allreduce_avg(xs_b, o_b, order, stream=side)

        def timed_side(fn, reps):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / reps

        reps = 20
        eager_ms = timed_side(per_bucket_sync, reps)
        graph = torch.cuda.CUDAGraph()
        per_bucket_sync()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            per_bucket_sync()
        graph_ms = timed_side(graph.replay, reps)
        del graph
        per_bucket = {"launches": plan.n_buckets, "python_loop_ms": round(eager_ms, 4),
                      "graph_replay_ms": round(graph_ms, 4), "one_launch_ms": round(ms_per_step, 4),
                      "one_launch_speedup_vs_graph": round(graph_ms / ms_per_step, 3)}
        log(f"per-bucket launches: {per_bucket}")

    # ---------------------------------------------------------------- MALL flushed
    # The same sync with a 512 MiB scratch buffer overwritten before each one,
    # so that nothing of the previous sync is left in the 256 MB MALL; each
    # sync bracketed by its own event pair (a few microseconds of event
    # overhead included).
    cold = None
    if not args.no_cold:
        scratch = torch.empty(1 << 27, dtype=torch.float32, device=dev)
        reps = min(args.steps, 50)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            scratch.fill_(1.0)
            a.record(stream)
            sync()
            b.record(stream)
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) for a, b in ev]
        cold = {"GBps_median": round(sync_bytes / (float(np.median(ts)) * 1e-3) / 1e9, 1),
                "GBps_best": round(sync_bytes / (min(ts) * 1e-3) / 1e9, 1),
                "ms_median": round(float(np.median(ts)), 5), "syncs": reps,
                "flush": "512 MiB written before every sync"}
        log(f"MALL flushed: {cold}")
        del scratch

    # ---------------------------------------------------------------- access-pattern ceiling
    # The same N input buffers read with the reduce's access pattern (N
    # non-temporal 16-byte loads per lane, one-wave blocks) with and without
    # the one store per lane, and no arithmetic: the ceiling of this pattern
    # on this machine, taken as the best over resident-block caps per CU (the
    # library caps its kernels the same way).  The probe's store covers the
    # input byte count, so it runs only when input and output elements have
    # the same size.
    ceiling = None
    if wl.in_bytes == wl.out_bytes and not args.no_ceiling:
        import ctypes
        probe = ctypes.CDLL(os.path.join(ROOT, "gradient_allreduce_averaging_amd", "libddp_probe.so"))
        probe.ddp_probe_stream.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        sink = torch.zeros(4, dtype=torch.int32, device=dev)
        nvec = P * wl.in_bytes // 16
        ptrs = (ctypes.c_void_p * N)(*[ctypes.c_void_p(f.data_ptr()) for f in flats])

        def probe_run(write, k):
            rc = probe.ddp_probe_stream(ptrs, N, ctypes.c_void_p(out.data_ptr()), nvec, write, k,
                                        ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(stream.cuda_stream))
            assert rc == 0, "probe launch failed"

        reps = min(args.steps, 50) if P < 10 ** 8 else 5
        res = {}
        for write in (1, 0):
            for k in (0, 16, 14, 12, 10, 9, 8, 7, 6):
                for _ in range(3):
                    probe_run(write, k)
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(reps):
                    probe_run(write, k)
                b.record(stream)
                torch.cuda.synchronize()
                ms = a.elapsed_time(b) / reps
                gbps = nvec * 16 * (N + write) / (ms * 1e-3) / 1e9
                if gbps > res.get(write, (0, 0))[0]:
                    res[write] = (gbps, k)
        ceiling = {"pattern_GBps": round(res[1][0], 1), "pattern_blocks_per_cu": res[1][1],
                   "read_only_GBps": round(res[0][0], 1), "read_only_blocks_per_cu": res[0][1],
                   "kernel_frac_of_pattern": round(achieved / res[1][0], 4),
                   "probe": f"{N} non-temporal 16-byte loads + 1 store per lane on the same "
                            "buffers, one-wave blocks, no arithmetic (read_only: without the "
                            "store); best over caps of 6..16 resident blocks per CU and none"}
        log(f"ceiling: {ceiling}")

    # ---------------------------------------------------------------- other order
    other = {}
    for o in ("seq", "ring"):
        if o == order:
            continue
        for _ in range(5):
            sync(o)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            sync(o)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        other[o] = {"ms_per_sync": round(ms, 5),
                    "GBps": round(sync_bytes / (ms * 1e-3) / 1e9, 1)}

    # ---------------------------------------------------------------- parity of the timed output
    parity = None
    cpu = None
    oplan, span, sampled = None, P, False
    if not args.no_cpu_baseline:
        import oracle
        if wl.two_bucket:
            oplan = oracle.plan_two_bucket(wl.numel, wl.regions)
        else:
            oplan = oracle.plan_cap(wl.numel, wl.bucket_cap_bytes, wl.in_bytes)
        sampled = wl.total * N * wl.in_bytes > (4 << 30)
        if sampled:
            # A bounded sample for the multi-GB workloads: the leading whole
            # buckets up to 4 GiB of inputs (a bucket's RING chunks depend on
            # its whole length).  The rate is the figure, labelled as
            # extrapolated; a first bucket above the budget skips it.
            keep = 0
            while keep < oplan.n_buckets and \
                    (oplan.bucket_base[keep] + oplan.bucket_len[keep]) * N * wl.in_bytes <= (4 << 30):
                keep += 1
            if keep == 0:
                log("cpu baseline skipped: the first bucket alone exceeds the 4 GiB sample budget")
                oplan = None
            else:
                span = oplan.bucket_base[keep - 1] + oplan.bucket_len[keep - 1]
                kept = [p for b in oplan.buckets[:keep] for p in b]
                sub, k = [], 0
                for b in oplan.buckets[:keep]:
                    sub.append(list(range(k, k + len(b))))
                    k += len(b)
                oplan = oracle.Plan([oplan.numel[p] for p in kept], sub)
    if oplan is not None:
        sync()
        torch.cuda.synchronize()
        got = out[:span].view(torch.int32 if tout == torch.float32 else torch.int16).cpu().numpy()
        host = [f[:span].view(torch.int32 if tin == torch.float32 else torch.int16).cpu().numpy()
                .view(np.float32 if tin == torch.float32 else np.uint16) for f in flats]
        sample_bytes = span * (N * wl.in_bytes + wl.out_bytes)
        reps, t_cpu = 0, 0.0
        want = None
        while reps == 0 or t_cpu < args.cpu_seconds:
            c0 = time.perf_counter()
            want = oracle.sync_avg(oplan, host, order, wl.dtype, wl.out_dtype)
            t_cpu += time.perf_counter() - c0
            reps += 1
        wv = want.view(np.int32 if tout == torch.float32 else np.int16)
        same = got == wv
        if tout == torch.float32:
            both_nan = np.isnan(got.view(np.float32)) & np.isnan(want)
        else:
            both_nan = np.zeros_like(same)
        parity = "bitwise equal to the CPU oracle" if bool((same | both_nan).all()) else \
            f"MISMATCH in {int((~(same | both_nan)).sum())} elements"
        cpu_model = "unknown"
        try:
            with open("/proc/cpuinfo") as f:
                cpu_model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
        except (OSError, StopIteration):
            pass
        what = (f"the first {oplan.n_buckets} bucket(s), {span} of {P} elements, of the {wl.name} "
                f"synchronisation; rate extrapolated to the whole" if sampled else
                f"the full {wl.name} synchronisation")
        cpu = {"value": round(sample_bytes * reps / t_cpu / 1e9, 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle", "host_cpu": cpu_model, "host_threads": os.cpu_count(),
               "sample": f"{what} ({order} order, N={N}), {reps} repetition(s), {t_cpu:.1f} s "
                         f"single-threaded C oracle"}
        if sampled:
            parity = parity + " (on the sampled buckets)"
        # context: a plain single-threaded host copy of 256 MiB (read + write bytes)
        src_h = np.ones(1 << 26, dtype=np.float32)
        dst_h = np.empty_like(src_h)
        np.copyto(dst_h, src_h)
        c0, n_cp = time.perf_counter(), 0
        while n_cp == 0 or time.perf_counter() - c0 < 1.0:
            np.copyto(dst_h, src_h)
            n_cp += 1
        cpu["host_copy_GBps"] = round(2 * src_h.nbytes * n_cp / (time.perf_counter() - c0) / 1e9, 2)
        del src_h, dst_h
        log(f"parity: {parity}; cpu oracle {cpu['value']} GB/s over {reps} reps; "
            f"host copy {cpu['host_copy_GBps']} GB/s")

        # The oracle on all of this process's host cores: SEQ order, every
        # bucket split into disjoint element ranges, one ctypes call per range
        # (the call releases the GIL).  SEQ has no index dependence, so the
        # split leaves every bit as it is; its result is checked against the
        # GPU's SEQ output of the same buffers.
        threads = min(16, len(os.sched_getaffinity(0)))
        pieces = []
        for base, ln in zip(oplan.bucket_base, oplan.bucket_len):
            step = max(1, -(-ln // threads))
            pieces += [(base + a, min(step, ln - a)) for a in range(0, ln, step)]
        seq_want = np.empty(span, dtype=np.float32 if tout == torch.float32 else np.uint16)

        def piece(pc):
            a, n = pc
            seq_want[a:a + n] = oracle.bucket_avg([h[a:a + n] for h in host], "seq",
                                                  wl.dtype, wl.out_dtype)

        from concurrent.futures import ThreadPoolExecutor
        reps_mt, t_mt = 0, 0.0
        with ThreadPoolExecutor(threads) as ex:
            while reps_mt == 0 or t_mt < args.cpu_seconds / 2:
                c0 = time.perf_counter()
                list(ex.map(piece, pieces))
                t_mt += time.perf_counter() - c0
                reps_mt += 1
        sync("seq")
        torch.cuda.synchronize()
        got_seq = out[:span].view(torch.int32 if tout == torch.float32 else torch.int16).cpu().numpy()
        sv = seq_want.view(got_seq.dtype)
        ok = got_seq == sv
        if tout == torch.float32:
            ok |= np.isnan(got_seq.view(np.float32)) & np.isnan(seq_want)
        cpu["all_cores"] = {
            "value": round(sample_bytes * reps_mt / t_mt / 1e9, 3), "unit": "GB/s", "cores": threads,
            "order": "seq", "parity_vs_gpu_seq": "bitwise equal" if bool(ok.all())
            else f"MISMATCH in {int((~ok).sum())} elements",
            "sample": f"{reps_mt} repetition(s) of {'the sample' if sampled else 'the full synchronisation'}"
                      f", {len(pieces)} element ranges on {threads} threads, {t_mt:.1f} s"}
        log(f"cpu oracle, {threads} threads (seq): {cpu['all_cores']['value']} GB/s; "
            f"{cpu['all_cores']['parity_vs_gpu_seq']}")

    # ---------------------------------------------------------------- copy layout
    copy_path = None
    if not args.no_copy_path and not wl.two_bucket and N * P * wl.in_bytes <= (16 << 30):
        # per-parameter gradients of every rank, holding the same values
        grads = [[torch.empty(n, dtype=tin, device=dev) for n in wl.numel] for _ in range(N)]
        binds = [ddp.bind_params(plan, grads[r]) for r in range(N)]
        for r in range(N):
            ddp.unflatten(plan, binds[r], flats[r], stream=stream)
        res = [torch.empty(n, dtype=tout, device=dev) for n in wl.numel]
        rbind = ddp.bind_params(plan, res)

        def full_step(st=stream):
            for r in range(N):
                ddp.flatten(plan, binds[r], flats[r], stream=st)
            ddp.sync_allreduce_avg(plan, flats, out, order, stream=st)
            ddp.unflatten(plan, rbind, out, stream=st)

        for _ in range(5):
            full_step()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        reps = max(10, args.steps // 4)
        tf = ts = tu = 0.0
        for _ in range(reps):
            e[0].record(stream)
            for r in range(N):
                ddp.flatten(plan, binds[r], flats[r], stream=stream)
            e[1].record(stream)
            sync()
            e[2].record(stream)
            ddp.unflatten(plan, rbind, out, stream=stream)
            e[3].record(stream)
            torch.cuda.synchronize()
            tf += e[0].elapsed_time(e[1])
            ts += e[1].elapsed_time(e[2])
            tu += e[2].elapsed_time(e[3])
        tf, ts, tu = tf / reps, ts / reps, tu / reps
        fb = 2 * N * P * wl.in_bytes
        ub = 2 * P * wl.out_bytes
        copy_path = {
            "ms_per_step": round(tf + ts + tu, 4),
            "flatten_ms": round(tf, 4), "flatten_GBps": round(fb / (tf * 1e-3) / 1e9, 1),
            "sync_ms": round(ts, 4),
            "unflatten_ms": round(tu, 4), "unflatten_GBps": round(ub / (tu * 1e-3) / 1e9, 1),
            "metric_GBps": round(sync_bytes / ((tf + ts + tu) * 1e-3) / 1e9, 1),
            "launches": N + 2}
        # the same step captured once into a HIP graph and replayed
        graph = torch.cuda.CUDAGraph()
        cap_stream = torch.cuda.Stream()
        cap_stream.wait_stream(stream)
        with torch.cuda.stream(cap_stream):
            with torch.cuda.graph(graph, stream=cap_stream):
                full_step(cap_stream)
        torch.cuda.synchronize()
        loop = {}
        for name, fn in (("eager", full_step), ("graph", graph.replay)):
            for _ in range(3):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            loop[name] = a.elapsed_time(b) / reps
        copy_path["eager_loop_ms_per_step"] = round(loop["eager"], 4)
        copy_path["graph_replay_ms_per_step"] = round(loop["graph"], 4)

        # the same step as one kernel over the per-parameter tensors
        ps = ddp.param_sync(plan, binds, rbind, order)
        for _ in range(5):
            ps(stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            ps(stream)
        b.record(stream)
        torch.cuda.synchronize()
        t_ps = a.elapsed_time(b) / reps
        chk = [torch.empty_like(t) for t in res]
        ddp.unflatten(plan, ddp.bind_params(plan, chk), out, stream=stream)   # out holds this sync
        torch.cuda.synchronize()
        same = all(torch.equal(x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32),
                               y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32))
                   for x, y in zip(res, chk))
        copy_path["param_sync"] = {
            "ms_per_step": round(t_ps, 4), "GBps": round(sync_bytes / (t_ps * 1e-3) / 1e9, 1),
            "speedup_vs_three_steps": round((tf + ts + tu) / t_ps, 2),
            "same_bits_as_three_steps": bool(same),
            "step": "every rank's per-parameter gradients averaged into per-parameter outputs "
                    "in one launch (ddp_param_sync_run)"}
        log(f"copy path: {copy_path}")
        del grads, binds, res, rbind, graph, ps, chk

    # ---------------------------------------------------------------- fused optimizer step
    # The average folded into a momentum-SGD step (ddp_sync_sgd_update) against
    # the unfused sequence it replaces: the synchronisation, then the optimizer
    # reading the averaged gradient back (torch's in-place ops).
    fused = None
    if not args.no_fused_sgd and wl.out_dtype == "f32":
        params = torch.empty(P, dtype=torch.float32, device=dev)
        W.device_normal_(params, 99, 7, 1.0)
        mbuf = torch.zeros(P, dtype=torch.float32, device=dev)
        lr, mu = 0.01, 0.9

        def fused_step():
            ddp.sync_sgd_update(plan, flats, params, lr, order, momentum_buf=mbuf, momentum=mu,
                                stream=stream)

        def unfused_step():
            sync()
            mbuf.mul_(mu).add_(out)
            params.add_(mbuf, alpha=-lr)

        res = {}
        for name, fn in (("fused", fused_step), ("unfused", unfused_step)):
            for _ in range(5):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(args.steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            res[name] = a.elapsed_time(b) / args.steps
        fb = N * P * wl.in_bytes + 4 * P * 4
        fused = {"ms": round(res["fused"], 5), "GBps": round(fb / (res["fused"] * 1e-3) / 1e9, 1),
                 "bytes": fb, "unfused_ms": round(res["unfused"], 5),
                 "speedup_vs_unfused": round(res["unfused"] / res["fused"], 3),
                 "step": "momentum SGD (mu 0.9) on f32 parameters; unfused = sync + torch mul_/add_"}
        # the same step on per-parameter tensors (gradients, parameters and
        # momentum buffers as autograd and the optimizer keep them)
        if N * P * wl.in_bytes <= (16 << 30):
            gviews = []
            for r in range(N):
                g = [torch.empty(n, dtype=tin, device=dev) for n in wl.numel]
                ddp.unflatten(plan, ddp.bind_params(plan, g), flats[r], stream=stream)
                gviews.append(g)
            pp = [torch.empty(n, dtype=torch.float32, device=dev).normal_() for n in wl.numel]
            pm = [torch.zeros(n, dtype=torch.float32, device=dev) for n in wl.numel]
            step = ddp.param_sgd(plan, [ddp.bind_params(plan, g) for g in gviews],
                                 ddp.bind_params(plan, pp), ddp.bind_params(plan, pm), None, order)
            for _ in range(5):
                step(lr, mu, stream)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(args.steps):
                step(lr, mu, stream)
            b.record(stream)
            torch.cuda.synchronize()
            t_p = a.elapsed_time(b) / args.steps
            fused["per_parameter"] = {
                "ms": round(t_p, 5), "GBps": round(fb / (t_p * 1e-3) / 1e9, 1),
                "step": "the same step on per-parameter gradients, parameters and momentum "
                        "(ddp_param_sgd_run)"}
            del gviews, pp, pm, step
        log(f"fused sgd: {fused}")
        del params, mbuf

    # ---------------------------------------------------------------- two-bucket overlap
    # The two-bucket plan of the same tensors: DEEP_COMM averaged on an update
    # stream while a GEMM (standing in for the first layer's backward) runs on
    # a compute stream; exposed = overlapped time - compute time.  Steps are
    # timed back to back with both streams joined at every step boundary.
    overlap = None
    if not args.no_overlap and wl.name == "resnet50":
        tb = ddp.plan_two_bucket(wl.numel, wl.regions, wl.dtype)
        (dl, db, _, _), (fl_, fb_, _, _) = tb.bucket(0), tb.bucket(1)
        mat_a = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
        mat_b = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
        comp, upd, tried = side_by_side_streams(torch)
        deep_in = [f[db:db + dl] for f in flats]
        deep_out = out[db:db + dl]

        def compute():
            with torch.cuda.stream(comp):
                torch.mm(mat_a, mat_b)

        def deep():
            ddp.bucket_allreduce_avg(deep_in, deep_out, order, stream=upd)

        def step_barrier():
            # a training step ends when both streams have: the next step's
            # backward needs the averaged gradients, and the next syncs the
            # next step's gradients
            e_comp, e_upd = torch.cuda.Event(), torch.cuda.Event()
            e_comp.record(comp)
            e_upd.record(upd)
            comp.wait_event(e_upd)
            upd.wait_event(e_comp)

        def timed(fns, reps=20):
            for _ in range(3):
                for f in fns:
                    f()
                step_barrier()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                for f in fns:
                    f()
                step_barrier()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / reps

        t_comp = timed([compute])
        overlap = {"plan": "two-bucket (DEEP_COMM %d, FIRST_COMM %d elements)" % (dl, fl_),
                   "compute_ms": round(t_comp, 4),
                   "compute": "bf16 GEMM 4096^3 on a second stream",
                   "streams": ("side by side (hardware queues checked; %d tried)" % tried
                               if tried else "not found side by side: results are serial")}
        # under both occupancy policies: the tuned cap reserves LDS that the
        # GEMM's blocks would need, "shared" leaves it free
        for policy in ("tuned", "shared"):
            ddp.set_occupancy(policy)
            t_deep = timed([deep])
            t_both = timed([compute, deep])
            overlap[policy] = {"deep_sync_ms": round(t_deep, 4), "overlapped_ms": round(t_both, 4),
                               "exposed_sync_ms": round(max(t_both - t_comp, 0.0), 4),
                               "hidden_fraction": round(1.0 - max(t_both - t_comp, 0.0) / t_deep, 3)}
        ddp.set_occupancy("tuned")

        # The bucket-by-bucket schedule of DDP ([DDP] 3.2, [TR24] 十一): bucket b
        # (cap plan, last layers first) is averaged on the update stream as
        # soon as a stand-in for the backward of its layers -- a bf16 GEMM
        # with FLOPs in proportion to the bucket's share of the parameters,
        # about 262 GFLOP in all (ResNet-50's backward at 32 images per GPU)
        # -- has finished on the compute stream.
        buckets = [plan.bucket(b) for b in range(plan.n_buckets)]
        ks = [max(64, int(round(7808 * ln / P / 64)) * 64) for ln, _, _, _ in buckets]
        lhs = [torch.randn(4096, k, device=dev, dtype=torch.bfloat16) for k in ks]
        rhs = [torch.randn(k, 4096, device=dev, dtype=torch.bfloat16) for k in ks]
        ready = [torch.cuda.Event() for _ in buckets]
        ins = [[f[base:base + ln] for f in flats] for ln, base, _, _ in buckets]
        outs_b = [out[base:base + ln] for ln, base, _, _ in buckets]

        def backward():
            with torch.cuda.stream(comp):
                for a, b, e in zip(lhs, rhs, ready):
                    torch.mm(a, b)
                    e.record(comp)

        def bucket_syncs(wait):
            for b in range(len(buckets)):
                if wait:
                    upd.wait_event(ready[b])
                ddp.bucket_allreduce_avg(ins[b], outs_b[b], order, stream=upd)

        t_bwd = timed([backward])
        gflop = sum(2 * 4096 * k * 4096 for k in ks) / 1e9
        overlap["schedule"] = {"buckets": len(buckets), "backward_gflop": round(gflop, 1),
                               "backward_ms": round(t_bwd, 4)}
        for policy in ("tuned", "shared"):
            ddp.set_occupancy(policy)
            t_syncs = timed([lambda: bucket_syncs(False)])
            t_sched = timed([backward, lambda: bucket_syncs(True)])
            overlap["schedule"][policy] = {
                "syncs_ms": round(t_syncs, 4), "serial_ms": round(t_bwd + t_syncs, 4),
                "overlapped_ms": round(t_sched, 4),
                "exposed_sync_ms": round(max(t_sched - t_bwd, 0.0), 4),
                "hidden_fraction": round(1.0 - max(t_sched - t_bwd, 0.0) / t_syncs, 3)}
        ddp.set_occupancy("tuned")

        # the same schedule on per-parameter gradients (as autograd leaves
        # them): bucket b of one ddp_param_sync per step, run when ready
        pg = []
        for r in range(N):
            g = [torch.empty(n, dtype=tin, device=dev) for n in wl.numel]
            ddp.unflatten(plan, ddp.bind_params(plan, g), flats[r], stream=stream)
            pg.append(g)
        pout = [torch.empty(n, dtype=tout, device=dev) for n in wl.numel]
        pps = ddp.param_sync(plan, [ddp.bind_params(plan, g) for g in pg],
                             ddp.bind_params(plan, pout), order)

        def param_syncs(wait):
            for b in range(len(buckets)):
                if wait:
                    upd.wait_event(ready[b])
                pps(upd, buckets=(b, 1))

        per_param = {"sync": "ddp_param_sync_run_buckets, one bucket per launch"}
        for policy in ("tuned", "shared"):
            ddp.set_occupancy(policy)
            t_psyncs = timed([lambda: param_syncs(False)])
            t_psched = timed([backward, lambda: param_syncs(True)])
            per_param[policy] = {
                "syncs_ms": round(t_psyncs, 4), "serial_ms": round(t_bwd + t_psyncs, 4),
                "overlapped_ms": round(t_psched, 4),
                "exposed_sync_ms": round(max(t_psched - t_bwd, 0.0), 4),
                "hidden_fraction": round(1.0 - max(t_psched - t_bwd, 0.0) / t_psyncs, 3)}
        ddp.set_occupancy("tuned")
        overlap["schedule"]["per_parameter"] = per_param
        del lhs, rhs, pg, pout, pps
        log(f"overlap: {overlap}")
        del mat_a, mat_b, tb

    # ---------------------------------------------------------------- rank sweep
    # The same plan averaged over N = 2..32 virtual ranks (N > 8 takes the
    # looped kernel): bandwidth against the number of concurrent streams.
    rank_sweep = None
    if not args.no_rank_sweep and wl.name == "resnet50":
        extra = []
        for r in range(N, 32):
            t = torch.empty(P, dtype=tin, device=dev)
            W.device_normal_(t, r, wl.stream, wl.sigma)
            extra.append(t)
        pool = flats + extra
        sweep_out = torch.empty(P, dtype=tout, device=dev)
        rank_sweep = {}
        for n in (2, 4, 6, 8, 9, 12, 16, 32):
            row = {}
            for o in ("ring", "seq"):
                call = ddp.make_sync(plan, pool[:n], sweep_out, o, stream=stream)
                for _ in range(3):
                    call()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(50):
                    call()
                b.record(stream)
                torch.cuda.synchronize()
                ms = a.elapsed_time(b) / 50
                row[o] = round((n * wl.in_bytes + wl.out_bytes) * P / (ms * 1e-3) / 1e9, 1)
            rank_sweep[str(n)] = row
        log(f"rank sweep (GB/s): {rank_sweep}")
        del extra, pool, sweep_out

    # ---------------------------------------------------------------- in place
    # The all-reduce as the pages run it, in place (send buffer == receive
    # buffer): the average overwrites rank 0's bucket buffer.  Runs after the
    # parity leg because it rewrites rank 0's gradients.
    in_place = {}
    for o in (() if args.no_in_place else ("ring", "seq")):
        call = ddp.make_sync(plan, flats, flats[0], o, stream=stream)
        for _ in range(3):
            call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        in_place[o] = {"ms_per_sync": round(ms, 5), "GBps": round(sync_bytes / (ms * 1e-3) / 1e9, 1)}
    log(f"in place: {in_place}")

    # ---------------------------------------------------------------- no_sync accumulation
    # M micro-steps: with no_sync each rank accumulates locally (M - 1
    # accumulates) and synchronises once; without it every micro-step also
    # synchronises.  Separate buffers keep the benchmark's inputs untouched.
    no_sync = None
    if not args.no_no_sync and 2 * N * P * wl.in_bytes <= (16 << 30):
        M = 4
        local = [f.clone() for f in flats]
        micro = [f.clone() for f in flats]

        def acc():
            ddp.accumulate(local, micro, stream=stream)

        def sync_local():
            ddp.sync_allreduce_avg(plan, local, out, order, stream=stream)

        res = {}
        for name, fn in (("acc", acc), ("sync", sync_local)):
            for _ in range(3):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(args.steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            res[name] = a.elapsed_time(b) / args.steps
        acc_bytes = 3 * N * P * wl.in_bytes
        no_sync = {"micro_steps": M, "accumulate_ms": round(res["acc"], 5),
                   "accumulate_GBps": round(acc_bytes / (res["acc"] * 1e-3) / 1e9, 1),
                   "no_sync_ms": round((M - 1) * res["acc"] + res["sync"], 5),
                   "sync_every_step_ms": round((M - 1) * res["acc"] + M * res["sync"], 5),
                   "syncs_saved": M - 1}
        log(f"no_sync: {no_sync}")
        del local, micro

    traffic = measured_traffic(wl.name, order, sync_bytes)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "pct_of_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {len(wl.params)} gradient tensors, "
                               f"{P} elements, {N} virtual ranks, {plan.n_buckets} buckets",
                   "virtual_ranks": N, "elements": P, "buckets": plan.n_buckets,
                   "bucket_cap_bytes": wl.bucket_cap_bytes,
                   "plan": "two-bucket" if wl.two_bucket else "cap",
                   "order": order, "grad_dtype": wl.dtype, "out_dtype": wl.out_dtype,
                   "grad_layout": "bucket view (gradients live in the per-rank flat buckets)",
                   "bytes_per_sync": sync_bytes,
                   "device": torch.cuda.get_device_name(0)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "reduce_fast (one launch per sync)",
                     "kernel_ms": round(kern_ms, 5),
                     "kernel_ms_source": "event pair around the K timed launches, / K",
                     "single_launch_ms_median": round(float(np.median(launch_ms)), 5),
                     "single_launch_ms_min": round(min(launch_ms), 5)},
        "per_bucket": per_bucket,
        "cold_mall": cold,
        "ceiling": ceiling,
        "cpu_baseline": cpu,
        "parity": parity,
        "other_orders": other,
        "copy_path": copy_path,
        "fused_sgd": fused,
        "in_place": in_place or None,
        "rank_sweep_GBps": rank_sweep,
        "overlap": overlap,
        "no_sync": no_sync,
        "env": run_environment(torch),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
