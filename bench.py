#!/usr/bin/env python3
"""Benchmark: bucketed gradient synchronisation on one MI355X.

Metric: effective HBM GB/s of one synchronisation, (N*P*b_in + P*b_out) /
t_sync, and its fraction of the 8 TB/s HBM peak.  A step is one whole
synchronisation of the workload: every bucket of the plan reduced over the N
virtual ranks in the fixed order, scaled by 1/N and written -- one launch of
ddp_sync_allreduce_avg.  Gradients sit in their bucket buffers (the
gradient-as-bucket-view layout), so flatten and unflatten are not needed in
the step; the ResNet-50 and many-small records also time the copy layout
(flatten every rank, sync, unflatten; the copies in bf16 as well) under
"copy_path".

The headline is GPT-1.3B (1.3 G f32 gradients, 8 virtual ranks, 146 buckets
of 25 MiB, ring order).  Every workload runs in a fresh child process of its
own; the parent never touches the GPU, idles --settle-seconds (20) before the
first child and --config-settle-seconds (10) before each further one
(buffers allocated within about 20 s of another process releasing tens of GB
of device memory were measured to stream 1-5 % slower).  The headline's
record is the line; the other workloads' records go under "configs",
GPT-1.3B's one-kernel sync over per-parameter tensors among them
("gpt1p3b:per-parameter").

Per workload: a declared clock ramp (back-to-back syncs for --ramp-ms, the
first K of them timed as "without_ramp"), W warm-up syncs, K timed syncs
(value, ms_per_step and the roofline), then
  cold_mall      the sync with the MALL flushed before each one
  ceiling        a probe of the reduce's bare access pattern
  other_orders   the other summation order
  cpu_baseline   the CPU oracle on all host cores and on one, with parity
  noalloc        the sync through the entry point that allocates nothing
and for ResNet-50 only (--extras): per_bucket, copy_path, fused_sgd,
overlap, rank_sweep_GBps, in_place, no_sync, small_means; for many-small
copy_path; for Llama-7B fused_sgd (the step on bf16 gradients); for tiny the
latency of a sync (Python call, prepared call, graph replay).

Prints ONE JSON line.  Only one GPU is used: --gpus above 1 exits with 2.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--configs a,b,...|none] [--order ring|seq] [--no-<section> ...]
       python bench.py --child --workload NAME [...]   (one workload, this process)
       python bench.py --child --layout per-parameter --workload NAME [...]
                       (the one-kernel sync over per-parameter tensors as the timed step)
       python bench.py --calibrate   (the plain-copy run that scales the HBM counters)
"""
import argparse
import hashlib
import json
import os
import re
import subprocess
import sys
import time
import types

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "effective HBM GB/s (N·P·bytes read + P written) and % of peak per sync"
CSRC = os.path.join(ROOT, "gradient_allreduce_averaging_amd", "csrc")
# the sources each timed kernel (the ones whose HBM counters are recorded) is
# built and launched from: its kernels and launches, the shared device code,
# the host helpers and the occupancy caps.  The flat reduce (bucket-view
# layout) and the per-parameter sync are hashed apart, so a change to one
# keeps the other's counter data.
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("common.hip", "device.h", "host.h", "reduce.hip")]
PARAMS_KERNEL_SOURCES = [os.path.join(CSRC, f)
                         for f in ("common.hip", "device.h", "host.h", "params.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha(layout="bucket-view"):
    """sha256[:16] of the layout's kernel sources (in name order) with
    comments and blank lines removed and each line stripped, so that only a
    change of code invalidates the counter data taken on it."""
    code = []
    for path in (PARAMS_KERNEL_SOURCES if layout == "per-parameter" else KERNEL_SOURCES):
        with open(path, encoding="utf-8") as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        lines = (re.sub(r"//.*", "", line).strip() for line in text.splitlines())
        code.append(os.path.basename(path) + "\n" + "\n".join(line for line in lines if line))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def traffic_key(workload, order, layout="bucket-view"):
    """The key of a workload's counter record in profiles/traffic.json."""
    return f"{workload}:per-parameter/{order}" if layout == "per-parameter" else \
        f"{workload}/{order}"


def measured_traffic(workload, order, layout="bucket-view"):
    """HBM bytes per launch from the committed rocprofv3 counter runs
    (profiles/traffic.json) and where they come from, or None and the reason
    when there are none for this kernel source.  The counters are not taken
    in this run."""
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None, "no counter file"
    key = traffic_key(workload, order, layout)
    rec = table.get(key)
    if not rec:
        return None, f"no counter run for {key}"
    sha = kernel_source_sha(layout)
    if rec.get("kernel_source_sha") != sha:
        return None, (f"counters taken on kernel source {rec.get('kernel_source_sha')}, not "
                      f"this one ({sha})")
    return rec.get("hbm_bytes_per_launch"), {
        "profile": rec.get("profile"), "kernel_source_sha": rec.get("kernel_source_sha"),
        "taken": rec.get("taken"), "read_bytes": rec.get("read_bytes"),
        "write_bytes": rec.get("write_bytes"),
        "how": "rocprofv3 FETCH_SIZE and WRITE_SIZE of the same kernel in committed runs, "
               "scaled as the profile states; not measured in this run"}


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


def hwmon_readings(torch):
    """Junction and memory (HBM) temperature in degrees C and board power in
    W of device 0, from its hwmon node in sysfs (empty when unreadable)."""
    import glob
    try:
        p = torch.cuda.get_device_properties(0)
        base = (f"/sys/bus/pci/devices/{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:"
                f"{p.pci_device_id:02x}.0/hwmon/hwmon*")
        def read(path):
            with open(path) as fh:
                return fh.read().strip()

        out = {}
        for d in glob.glob(base):
            for f in glob.glob(d + "/temp*_label"):
                out[f"{read(f)}_C"] = int(read(f.replace("_label", "_input"))) / 1000
            if os.path.exists(d + "/power1_input"):
                out["power_W"] = int(read(d + "/power1_input")) / 1e6
        return out
    except (OSError, AttributeError, ValueError):
        return {}


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


def stream_ms(c, fn, reps, warm=3, settle=False):
    """Average ms per call of fn: `warm` untimed calls, then `reps` calls
    between one event pair on the launch stream (after a device-wide
    synchronisation when `settle`)."""
    torch = c.torch
    for _ in range(warm):
        fn()
    if settle:
        torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(c.stream)
    for _ in range(reps):
        fn()
    b.record(c.stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def gbps(nbytes, ms):
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


DEFAULT_CONFIGS = ("resnet50,many_small,tiny,gpt1p3b_two_bucket,gpt1p3b:per-parameter,"
                   "llama7b")


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt1p3b",
                    help="the headline workload (default gpt1p3b: GPT-1.3B, 146 buckets, N=8)")
    ap.add_argument("--configs", default=DEFAULT_CONFIGS,
                    help="the other workloads measured after the headline, each in a fresh child "
                         "process, comma-separated; NAME:per-parameter times the one-kernel sync over "
                         "per-parameter tensors ('none' for the headline alone)")
    ap.add_argument("--child", action="store_true",
                    help="measure --workload in this process and print its JSON line (what the "
                         "parent runs per workload; the parent itself never touches the GPU)")
    ap.add_argument("--extras", default=None, choices=["on", "off"],
                    help="the legs beyond the metric (per-bucket launches, copy path, fused SGD, "
                         "overlap, rank sweep, in place, no_sync, small means); default: on for "
                         "resnet50 only")
    ap.add_argument("--order", default=None, choices=["ring", "seq"],
                    help="summation order of the timed sync (default: ring, or the workload's only "
                         "order: seq for tiny)")
    ap.add_argument("--ramp-ms", type=float, default=300.0,
                    help="time-based clock ramp: syncs run back to back for at least this long "
                         "before the counted warm-up (declared in the line with the rate of the "
                         "first K syncs, i.e. the result without it)")
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
    ap.add_argument("--layout", default="bucket-view", choices=["bucket-view", "per-parameter"],
                    help="bucket-view: the timed step reads the per-rank flat buckets "
                         "(ddp_sync_allreduce_avg); per-parameter: it reads every rank's "
                         "per-parameter tensors in one kernel (ddp_param_sync_run), and only the "
                         "timed step, the flushed-MALL leg, the other order and parity run")
    ap.add_argument("--settle-seconds", type=float, default=20.0,
                    help="idle pause before the first child starts (0 to skip): buffers allocated "
                         "within about 20 s of another process releasing tens of GB of device "
                         "memory were measured to stream 1-5 %% slower for as long as they live")
    ap.add_argument("--config-settle-seconds", type=float, default=10.0,
                    help="idle pause before each further child (after the previous one released "
                         "its buffers)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle time of the headline (half on one thread, half on all cores)")
    ap.add_argument("--config-cpu-seconds", type=float, default=4.0,
                    help="CPU oracle time of each further workload")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 10 times (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def setup(args):
    """The workload's plan, its N rank buffers (seeded synthetic gradients,
    resident in HBM) and output, and the prepared synchronisation calls."""
    import numpy as np
    import torch

    import gradient_allreduce_averaging_amd as ddp
    import workloads as W

    c = types.SimpleNamespace(args=args, np=np, torch=torch, ddp=ddp, W=W)
    c.dev = torch.device("cuda:0")
    c.wl = wl = W.workload(args.workload)
    c.order = args.order or ("ring" if "ring" in wl.orders else wl.orders[0])
    c.N = N = wl.n_ranks
    if wl.two_bucket:
        c.plan = ddp.plan_two_bucket(wl.numel, wl.regions, wl.dtype)
    else:
        c.plan = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, wl.dtype)
    c.P = P = c.plan.total
    c.tin = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    c.tout = torch.float32 if wl.out_dtype == "f32" else torch.bfloat16
    log(f"workload {wl.name}: N={N} P={P} buckets={c.plan.n_buckets} order={c.order} "
        f"{wl.dtype}->{wl.out_dtype}")
    c.plan.prepare()
    c.stream = torch.cuda.current_stream()
    c.sync_bytes = wl.sync_bytes()
    if args.layout == "per-parameter":
        setup_per_parameter(c)
        return c
    c.flats = []
    for r in range(N):
        t = torch.empty(P, dtype=c.tin, device=c.dev)
        W.device_normal_(t, r, wl.stream, wl.sigma)
        c.flats.append(t)
    c.out = torch.empty(P, dtype=c.tout, device=c.dev)
    prepared = {o: ddp.make_sync(c.plan, c.flats, c.out, o, stream=c.stream) for o in ("seq", "ring")}

    def sync(o=c.order):
        prepared[o]()

    c.sync = sync
    return c


def setup_per_parameter(c):
    """Per-parameter gradient tensors of every rank, as autograd leaves them
    (the same distribution, seeded per rank and tensor), per-parameter
    outputs, and the one-kernel sync (ddp_param_sync_run).  Nothing large is
    allocated and freed before the timed steps."""
    torch, ddp, plan, wl = c.torch, c.ddp, c.plan, c.wl
    c.grads = []
    for r in range(c.N):
        g = [torch.empty(n, dtype=c.tin, device=c.dev) for n in wl.numel]
        for p, t in enumerate(g):
            c.W.device_normal_(t, r * 100_003 + p, wl.stream, wl.sigma)
        c.grads.append(g)
    c.pout = [torch.empty(n, dtype=c.tout, device=c.dev) for n in wl.numel]
    binds = [ddp.bind_params(plan, g) for g in c.grads]
    obind = ddp.bind_params(plan, c.pout)
    prepared = {o: ddp.param_sync(plan, binds, obind, o) for o in ("seq", "ring")}

    def sync(o=c.order):
        prepared[o](c.stream)

    c.sync = sync


def leg_parity_per_parameter(c):
    """Per-parameter layout: the timed outputs against the flat sync of the
    same values (flatten every rank, ddp_sync_allreduce_avg, unflatten), bit
    for bit, where the flat copies fit beside the tensors (inputs up to
    16 GB); the GPU tests check every workload against the oracle."""
    torch, ddp, plan, wl = c.torch, c.ddp, c.plan, c.wl
    if c.N * c.P * wl.in_bytes > (16 << 30):
        return ("not checked here (inputs above 16 GB); tests/test_gpu_full_size.py compares every "
                "element with the oracle")
    c.sync()
    flats = [torch.empty(c.P, dtype=c.tin, device=c.dev) for _ in range(c.N)]
    for g, f in zip(c.grads, flats):
        ddp.flatten(plan, ddp.bind_params(plan, g), f, stream=c.stream)
    out = torch.empty(c.P, dtype=c.tout, device=c.dev)
    ddp.sync_allreduce_avg(plan, flats, out, c.order, stream=c.stream)
    want = [torch.empty_like(t) for t in c.pout]
    ddp.unflatten(plan, ddp.bind_params(plan, want), out, stream=c.stream)
    torch.cuda.synchronize()
    bits = torch.int16 if c.tout == torch.bfloat16 else torch.int32
    same = all(torch.equal(x.view(bits), y.view(bits)) for x, y in zip(c.pout, want))
    return ("bitwise equal to flatten + sync + unflatten of the same values" if same
            else "MISMATCH against flatten + sync + unflatten")


def timed_steps(c):
    """The metric.  First a declared, time-based clock ramp: syncs back to
    back for at least --ramp-ms, of which the first K are timed between one
    event pair (the result without a ramp).  Then W untimed warm-up syncs and
    K timed back-to-back syncs, wall clock between two synchronisations, with
    one event pair around the loop on the launch stream.  Then the same K
    steps with each launch between its own event pair (these add the event
    overhead of a few microseconds to each)."""
    torch, args = c.torch, c.args
    K = args.steps
    torch.cuda.synchronize()
    first_a, first_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_ramp0 = time.perf_counter()
    first_a.record(c.stream)
    for _ in range(K):
        c.sync()
    first_b.record(c.stream)
    n_ramp = K
    torch.cuda.synchronize()
    while (time.perf_counter() - t_ramp0) * 1e3 < args.ramp_ms:
        for _ in range(4):
            c.sync()
        n_ramp += 4
        torch.cuda.synchronize()
    ramp_ms = (time.perf_counter() - t_ramp0) * 1e3
    first_ms = first_a.elapsed_time(first_b) / K
    c.ramp = {"min_ms": args.ramp_ms, "ms": round(ramp_ms, 2), "syncs": n_ramp,
              "without_ramp": {"syncs": K, "kernel_ms": round(first_ms, 5),
                               "GBps": gbps(c.sync_bytes, first_ms),
                               "how": "the first K syncs of the process, one event pair"}}
    for _ in range(args.warmup):
        c.sync()
    loop_a, loop_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop_a.record(c.stream)
    for _ in range(K):
        c.sync()
    loop_b.record(c.stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    c.ms_per_step = (t1 - t0) * 1e3 / K
    # The reduce kernel's average launch duration: the event pair around the
    # timed loop on the launch stream, over K back-to-back launches (one
    # kernel per step, so this is the kernel plus the launch gap).
    c.kern_ms = loop_a.elapsed_time(loop_b) / K
    c.value = c.sync_bytes / (c.ms_per_step * 1e-3) / 1e9
    c.achieved = c.sync_bytes / (c.kern_ms * 1e-3) / 1e9
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for a, b in ev:
        a.record(c.stream)
        c.sync()
        b.record(c.stream)
    torch.cuda.synchronize()
    c.launch_ms = [a.elapsed_time(b) for a, b in ev]
    log(f"{c.wl.name}: ramp {ramp_ms:.0f} ms ({n_ramp} syncs; first {K}: {first_ms * 1e3:.1f} us "
        f"each); {c.ms_per_step * 1e3:.1f} us/step wall, {c.kern_ms * 1e3:.1f} us/step on the "
        f"stream ({c.achieved:.0f} GB/s); single launches between events: median "
        f"{c.np.median(c.launch_ms) * 1e3:.1f} us, min {min(c.launch_ms) * 1e3:.1f} us")


def leg_per_bucket(c):
    """The same sync as DDP issues it, one all-reduce call per bucket
    (ddp_bucket_allreduce_avg on each bucket's sub-ranges): driven from
    Python, and replayed from a HIP graph that captured those launches.
    Against the one-launch sync this is the launch overhead it saves."""
    torch, ddp, plan = c.torch, c.ddp, c.plan
    if c.args.no_per_bucket or not 1 < plan.n_buckets <= 4096 or c.P >= 10 ** 9:
        return None
    spans = [plan.bucket(b)[:2] for b in range(plan.n_buckets)]
    ins_b = [[f[base:base + ln] for f in c.flats] for ln, base in spans]
    outs_b = [c.out[base:base + ln] for ln, base in spans]
    side = torch.cuda.Stream()

    def per_bucket_sync():
        for xs_b, o_b in zip(ins_b, outs_b):
            ddp.bucket_allreduce_avg(xs_b, o_b, c.order, stream=side)

    def timed_side(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / reps

    eager_ms = timed_side(per_bucket_sync, 20)
    graph = torch.cuda.CUDAGraph()
    per_bucket_sync()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        per_bucket_sync()
    graph_ms = timed_side(graph.replay, 20)
    del graph
    res = {"launches": plan.n_buckets, "python_loop_ms": round(eager_ms, 4),
           "graph_replay_ms": round(graph_ms, 4), "one_launch_ms": round(c.ms_per_step, 4),
           "one_launch_speedup_vs_graph": round(graph_ms / c.ms_per_step, 3)}
    log(f"per-bucket launches: {res}")
    return res


def leg_cold_mall(c):
    """The sync with nothing of the previous one left in the 256 MB MALL:
    K times (overwrite a 512 MiB scratch buffer, sync) between one event
    pair, minus K overwrites alone between another, divided by K -- the same
    back-to-back form as the headline, so the two differ only by MALL reuse.
    Three trials; the median is reported."""
    torch, np = c.torch, c.np
    if c.args.no_cold or c.sync_bytes < (64 << 20):
        return None   # a sync of a few KB lives in the caches whatever is flushed
    scratch = torch.empty(1 << 27, dtype=torch.float32, device=c.dev)
    reps = max(5, min(c.args.steps, 50))

    def pair(with_sync):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(c.stream)
        for _ in range(reps):
            scratch.fill_(1.0)
            if with_sync:
                c.sync()
        b.record(c.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    pair(True)
    per_sync, flush = [], []
    for _ in range(3):
        both, alone = pair(True), pair(False)
        per_sync.append((both - alone) / reps)
        flush.append(alone / reps)
    ms = float(np.median(per_sync))
    res = {"GBps": gbps(c.sync_bytes, ms), "ms_per_sync": round(ms, 5),
           "frac_of_peak": round(c.sync_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
           "vs_back_to_back": round(c.kern_ms / ms, 4),
           "flush_ms": round(float(np.median(flush)), 5), "syncs": reps, "trials": 3,
           "how": "event pair around K x (512 MiB overwrite + sync) minus one around K "
                  "overwrites alone, / K; median of 3 trials"}
    del scratch
    log(f"MALL flushed: {res}")
    return res


def leg_ceiling(c):
    """The same N input buffers read with the reduce's access pattern (N
    non-temporal 16-byte loads per lane, one-wave blocks) with and without
    the one store per lane, and no arithmetic: the ceiling of this pattern on
    this box, taken as the best over resident-block caps per CU (the library
    caps its kernels the same way).  The probe's store covers the input byte
    count, so it runs only when input and output elements have the same
    size."""
    import ctypes
    torch, wl, N = c.torch, c.wl, c.N
    if wl.in_bytes != wl.out_bytes or c.args.no_ceiling or c.sync_bytes < (64 << 20):
        return None   # (a sync of a few KB is latency-bound: no bandwidth ceiling to compare)
    probe = ctypes.CDLL(os.path.join(ROOT, "gradient_allreduce_averaging_amd", "libddp_probe.so"))
    probe.ddp_probe_stream.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device=c.dev)
    nvec = c.P * wl.in_bytes // 16
    ptrs = (ctypes.c_void_p * N)(*[ctypes.c_void_p(f.data_ptr()) for f in c.flats])

    def probe_run(write, k):
        rc = probe.ddp_probe_stream(ptrs, N, ctypes.c_void_p(c.out.data_ptr()), nvec, write, k,
                                    ctypes.c_void_p(sink.data_ptr()),
                                    ctypes.c_void_p(c.stream.cuda_stream))
        assert rc == 0, "probe launch failed"

    reps = min(c.args.steps, 50) if c.P < 10 ** 8 else 5
    best = {}
    for write in (1, 0):
        for k in (0, 16, 14, 12, 10, 9, 8, 7, 6):
            ms = stream_ms(c, lambda: probe_run(write, k), reps)
            rate = nvec * 16 * (N + write) / (ms * 1e-3) / 1e9
            if rate > best.get(write, (0, 0))[0]:
                best[write] = (rate, k)
    res = {"pattern_GBps": round(best[1][0], 1), "pattern_blocks_per_cu": best[1][1],
           "read_only_GBps": round(best[0][0], 1), "read_only_blocks_per_cu": best[0][1],
           "kernel_frac_of_pattern": round(c.achieved / best[1][0], 4),
           "probe": f"{N} non-temporal 16-byte loads + 1 store per lane on the same "
                    "buffers, one-wave blocks, no arithmetic (read_only: without the "
                    "store); best over caps of 6..16 resident blocks per CU and none"}
    log(f"ceiling: {res}")
    return res


def leg_other_orders(c):
    res = {}
    for o in ("seq", "ring"):
        if o == c.order:
            continue
        ms = stream_ms(c, lambda: c.sync(o), c.args.steps, warm=5)
        res[o] = {"ms_per_sync": round(ms, 5), "GBps": gbps(c.sync_bytes, ms)}
    return res


SAMPLE_INPUT_BYTES = 4 << 30


def oracle_sample(c, oracle):
    """The runs of elements the CPU oracle computes: the whole plan, or for
    the multi-GB workloads a bounded sample -- the leading buckets up to
    4 GiB of inputs, the last one cut short where the budget ends (a piece
    keeps its position in its bucket, so its ring chunks are the whole
    bucket's).  Returns [(flat start, bucket length, position in bucket,
    count)] and whether it is a sample."""
    wl, N = c.wl, c.N
    if wl.two_bucket:
        oplan = oracle.plan_two_bucket(wl.numel, wl.regions)
    else:
        oplan = oracle.plan_cap(wl.numel, wl.bucket_cap_bytes, wl.in_bytes)
    budget = SAMPLE_INPUT_BYTES // (N * wl.in_bytes)   # elements
    runs, left = [], budget
    for base, ln in zip(oplan.bucket_base, oplan.bucket_len):
        if ln == 0:
            continue
        n = min(ln, left)
        if n <= 0:
            break
        runs.append((base, ln, 0, n))
        left -= n
    return runs, sum(r[3] for r in runs) < c.P


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        return "unknown"


def leg_parity_and_cpu(c, cpu_seconds):
    """Parity of the timed output against the CPU oracle, and the oracle's
    rate on the host: the oracle's piece form (each element folded at its
    position in its bucket) over the same runs of elements, split into
    disjoint ranges on all of this process's host cores (the C call releases
    the GIL, and the split leaves every bit as it is), then on one thread.
    Half of cpu_seconds each."""
    if c.args.no_cpu_baseline:
        return None, None
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    torch, np, wl, N, order = c.torch, c.np, c.wl, c.N, c.order
    runs, sampled = oracle_sample(c, oracle)
    span = sum(n for _, _, _, n in runs)
    f32_in, f32_out = c.tin == torch.float32, c.tout == torch.float32
    in_np, out_np = (np.float32 if f32_in else np.uint16), (np.float32 if f32_out else np.uint16)
    c.sync()
    torch.cuda.synchronize()

    def host(t, a, n):
        return t[a:a + n].view(torch.int32 if t.dtype == torch.float32 else torch.int16) \
            .cpu().numpy().view(np.float32 if t.dtype == torch.float32 else np.uint16)

    xs = [np.concatenate([host(f, a, n) for a, _, _, n in runs]) for f in c.flats]
    got = np.concatenate([host(c.out, a, n) for a, _, _, n in runs])
    # threads: the CPUs this process may use (at most 16, the box's share),
    # one per million elements at least
    threads = max(1, min(16, len(os.sched_getaffinity(0)), span >> 20))
    pieces, k = [], 0          # (offset in the sample, bucket length, position, count)
    for _, ln, pos, n in runs:
        step = max(1, -(-n // threads))
        pieces += [(k + s, ln, pos + s, min(step, n - s)) for s in range(0, n, step)]
        k += n
    want = np.empty(span, dtype=out_np)

    def piece(pc):
        k0, ln, pos, n = pc
        oracle.bucket_range_avg([x[k0:k0 + n] for x in xs], ln, pos, order, wl.dtype,
                                wl.out_dtype, out=want[k0:k0 + n])

    sample_bytes = span * (N * wl.in_bytes + wl.out_bytes)

    def timed_runs(ex, budget):
        reps, t = 0, 0.0
        while reps == 0 or t < budget:
            t0 = time.perf_counter()
            if ex is None:
                for pc in pieces:
                    piece(pc)
            else:
                list(ex.map(piece, pieces))
            t += time.perf_counter() - t0
            reps += 1
        return reps, t

    with ThreadPoolExecutor(threads) as ex:
        reps_mt, t_mt = timed_runs(ex, cpu_seconds / 2)
    same = got.view(np.uint32 if f32_out else np.uint16) == want.view(np.uint32 if f32_out
                                                                       else np.uint16)
    if f32_out:
        same |= np.isnan(got) & np.isnan(want)
    parity = "bitwise equal to the CPU oracle" if bool(same.all()) else \
        f"MISMATCH in {int((~same).sum())} elements"
    reps_1, t_1 = timed_runs(None, cpu_seconds / 2)
    what = (f"the leading {span} of {c.P} elements ({len(runs)} bucket(s), the last one cut at "
            f"4 GiB of inputs) of the {wl.name} synchronisation; rate extrapolated to the whole"
            if sampled else f"the full {wl.name} synchronisation")
    cpu = {"value": round(sample_bytes * reps_mt / t_mt / 1e9, 3), "unit": "GB/s",
           "cores": threads, "kind": "oracle", "order": order,
           "host_cpu": _cpu_model(), "host_threads": os.cpu_count(),
           "sample": f"{what} ({order} order, N={N}): {reps_mt} repetition(s) in "
                     f"{t_mt:.1f} s, {len(pieces)} element ranges on {threads} threads "
                     f"(oracle.bucket_range_avg)",
           "single_thread": {"value": round(sample_bytes * reps_1 / t_1 / 1e9, 3),
                             "unit": "GB/s", "cores": 1,
                             "sample": f"the same, {reps_1} repetition(s) in {t_1:.1f} s"}}
    if sampled:
        parity = parity + f" (on the sampled {span} elements)"
    # context: a plain single-threaded host copy of 256 MiB (read + write bytes)
    src_h = np.ones(1 << 26, dtype=np.float32)
    dst_h = np.empty_like(src_h)
    np.copyto(dst_h, src_h)
    c0, n_cp = time.perf_counter(), 0
    while n_cp == 0 or time.perf_counter() - c0 < 1.0:
        np.copyto(dst_h, src_h)
        n_cp += 1
    cpu["host_copy_GBps"] = round(2 * src_h.nbytes * n_cp / (time.perf_counter() - c0) / 1e9, 2)
    log(f"{wl.name} parity: {parity}; cpu oracle {cpu['value']} GB/s on {threads} threads, "
        f"{cpu['single_thread']['value']} GB/s on one; host copy {cpu['host_copy_GBps']} GB/s")
    return parity, cpu


def rank_grads(c):
    """Per-parameter gradient tensors of every rank holding the values of the
    rank buffers, as autograd would leave them."""
    grads = []
    for r in range(c.N):
        g = [c.torch.empty(n, dtype=c.tin, device=c.dev) for n in c.wl.numel]
        c.ddp.unflatten(c.plan, c.ddp.bind_params(c.plan, g), c.flats[r], stream=c.stream)
        grads.append(g)
    return grads


def copy_ceiling(c, flats=None, out=None, esize=None):
    """A plain copy of one rank buffer (the bytes one flatten or unflatten
    launch moves), one launch per rank back to back, through the probe's
    one-load-one-store pattern (non-temporal 16-byte accesses, one-wave
    blocks): the ceiling of a copy of this size on this machine, best over
    resident-block caps.  Defaults: the workload's rank buffers and output."""
    import ctypes
    torch, N, wl = c.torch, c.N, c.wl
    if flats is None:
        if wl.in_bytes != wl.out_bytes:
            return None
        flats, out, esize = c.flats, c.out, wl.in_bytes
    probe = ctypes.CDLL(os.path.join(ROOT, "gradient_allreduce_averaging_amd", "libddp_probe.so"))
    probe.ddp_probe_stream.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device=c.dev)
    nvec = c.P * esize // 16
    srcs = [(ctypes.c_void_p * 1)(ctypes.c_void_p(f.data_ptr())) for f in flats]

    def copies(k):
        for src in srcs:
            rc = probe.ddp_probe_stream(src, 1, ctypes.c_void_p(out.data_ptr()), nvec, 1, k,
                                        ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(c.stream.cuda_stream))
            assert rc == 0, "probe launch failed"

    best = (0.0, 0)
    for k in (0, 4, 5, 6, 7, 8):
        ms = stream_ms(c, lambda: copies(k), 10, settle=True)
        rate = 2 * N * nvec * 16 / (ms * 1e-3) / 1e9
        best = max(best, (rate, k))
    return {"GBps": round(best[0], 1), "blocks_per_cu": best[1],
            "probe": f"{N} launches, each a plain copy of one rank buffer ({nvec * 16} B) with the "
                     "one-load-one-store pattern, back to back; best over caps of 4..8 resident "
                     "blocks per CU and none"}


def carved_view_rates(c, binds, reps, t_unflatten, t_param_sync):
    """The outputs as views carved back to back, in registration order, out
    of one buffer one element past an aligned allocation (a flat gradient
    buffer viewed per parameter): neighbouring parameters then share 16-byte
    pieces of storage.  Unflatten into them and the one-kernel sync writing
    into them, timed as the separate tensors are, with the same bits."""
    torch, ddp, plan, wl = c.torch, c.ddp, c.plan, c.wl
    big = torch.empty(c.P + 1, dtype=c.tout, device=c.dev)
    views, o = [], 1
    for n in wl.numel:
        views.append(big[o:o + n])
        o += n
    vb = ddp.bind_params(plan, views)
    tu = stream_ms(c, lambda: ddp.unflatten(plan, vb, c.out, stream=c.stream), reps, settle=True)
    ps = ddp.param_sync(plan, binds, vb, c.order)
    t_ps = stream_ms(c, lambda: ps(c.stream), reps, warm=5, settle=True)
    chk = [torch.empty_like(v) for v in views]
    ddp.unflatten(plan, ddp.bind_params(plan, chk), c.out, stream=c.stream)
    torch.cuda.synchronize()
    same = all(torch.equal(x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32),
                           y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32))
               for x, y in zip(views, chk))
    res = {"unflatten_ms": round(tu, 4), "unflatten_GBps": gbps(2 * c.P * wl.out_bytes, tu),
           "unflatten_vs_separate_tensors": round(t_unflatten / tu, 4),
           "param_sync_ms": round(t_ps, 4), "param_sync_GBps": gbps(c.sync_bytes, t_ps),
           "param_sync_vs_separate_tensors": round(t_param_sync / t_ps, 4),
           "same_bits_as_unflatten": bool(same),
           "layout": "outputs carved back to back out of one buffer, 1 element past its start"}
    del big, views, vb, ps, chk
    torch.cuda.empty_cache()
    return res


def copy_rates_bf16(c, reps):
    """Flatten and unflatten of the same parameter sizes in bf16: per-rank
    bf16 tensors, a bf16 plan with the workload's cap, each copy timed back
    to back (K repetitions between one event pair), GB/s by the bytes it
    moves; the plain copy of one bf16 rank buffer beside them.  The
    tensors are filled by unflattening the rank buffers, so flattening them
    again must give those buffers back bit for bit."""
    torch, ddp, wl, N = c.torch, c.ddp, c.wl, c.N
    plan = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, "bf16")
    gen = torch.Generator(device=c.dev)
    gen.manual_seed(5)
    flats = [torch.empty(c.P, dtype=torch.bfloat16, device=c.dev).normal_(0, 1e-3, generator=gen)
             for _ in range(N)]
    grads = [[torch.empty(n, dtype=torch.bfloat16, device=c.dev) for n in wl.numel]
             for _ in range(N)]
    binds = [ddp.bind_params(plan, g) for g in grads]
    for r in range(N):
        ddp.unflatten(plan, binds[r], flats[r], stream=c.stream)
    want = [f.clone() for f in flats]

    def flatten_all():
        for r in range(N):
            ddp.flatten(plan, binds[r], flats[r], stream=c.stream)

    def unflatten_one():
        ddp.unflatten(plan, binds[0], flats[0], stream=c.stream)

    tf = stream_ms(c, flatten_all, reps, settle=True)
    tu = stream_ms(c, unflatten_one, reps, settle=True)
    torch.cuda.synchronize()
    same = all(torch.equal(f.view(torch.int16), w.view(torch.int16)) for f, w in zip(flats, want))
    out = {"flatten_ms": round(tf, 4), "flatten_GBps": gbps(2 * N * c.P * 2, tf),
           "unflatten_ms": round(tu, 4), "unflatten_GBps": gbps(2 * c.P * 2, tu),
           "flatten_gives_the_rank_buffers_back": bool(same)}
    scratch = torch.empty(c.P, dtype=torch.bfloat16, device=c.dev)
    ceil = copy_ceiling(c, flats, scratch, 2)
    if ceil:
        out["copy_ceiling"] = ceil
        out["flatten_frac_of_copy_ceiling"] = round(out["flatten_GBps"] / ceil["GBps"], 4)
        out["unflatten_frac_of_copy_ceiling"] = round(out["unflatten_GBps"] / ceil["GBps"], 4)
    del flats, grads, binds, want, scratch
    torch.cuda.empty_cache()
    return out


def leg_copy_path(c):
    """The copy layout: flatten every rank, sync, unflatten (timed step by
    step, as an eager loop and replayed from a HIP graph), and the same step
    as one kernel over the per-parameter tensors."""
    torch, ddp, plan, wl, N = c.torch, c.ddp, c.plan, c.wl, c.N
    if c.args.no_copy_path or wl.two_bucket or N * c.P * wl.in_bytes > (16 << 30):
        return None
    grads = rank_grads(c)
    binds = [ddp.bind_params(plan, g) for g in grads]
    res = [torch.empty(n, dtype=c.tout, device=c.dev) for n in wl.numel]
    rbind = ddp.bind_params(plan, res)

    def full_step(st=c.stream):
        for r in range(N):
            ddp.flatten(plan, binds[r], c.flats[r], stream=st)
        ddp.sync_allreduce_avg(plan, c.flats, c.out, c.order, stream=st)
        ddp.unflatten(plan, rbind, c.out, stream=st)

    for _ in range(5):
        full_step()
    reps = max(10, c.args.steps // 4)

    def flatten_all():
        for r in range(N):
            ddp.flatten(plan, binds[r], c.flats[r], stream=c.stream)

    def unflatten_one():
        ddp.unflatten(plan, rbind, c.out, stream=c.stream)

    # each step back to back, K times between one event pair, as the
    # headline times the sync
    tf = stream_ms(c, flatten_all, reps, settle=True)
    ts = stream_ms(c, c.sync, reps, settle=True)
    tu = stream_ms(c, unflatten_one, reps, settle=True)
    out = {"ms_per_step": round(tf + ts + tu, 4),
           "flatten_ms": round(tf, 4), "flatten_GBps": gbps(2 * N * c.P * wl.in_bytes, tf),
           "sync_ms": round(ts, 4),
           "unflatten_ms": round(tu, 4), "unflatten_GBps": gbps(2 * c.P * wl.out_bytes, tu),
           "metric_GBps": gbps(c.sync_bytes, tf + ts + tu),
           "launches": N + 2,
           "timing": "each step K times back to back between one event pair"}
    ceil = copy_ceiling(c)
    if ceil:
        out["copy_ceiling"] = ceil
        out["flatten_frac_of_copy_ceiling"] = round(out["flatten_GBps"] / ceil["GBps"], 4)
        out["unflatten_frac_of_copy_ceiling"] = round(out["unflatten_GBps"] / ceil["GBps"], 4)
    # the same step captured once into a HIP graph and replayed
    graph = torch.cuda.CUDAGraph()
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(c.stream)
    with torch.cuda.stream(cap_stream):
        with torch.cuda.graph(graph, stream=cap_stream):
            full_step(cap_stream)
    torch.cuda.synchronize()
    out["eager_loop_ms_per_step"] = round(stream_ms(c, full_step, reps, settle=True), 4)
    out["graph_replay_ms_per_step"] = round(stream_ms(c, graph.replay, reps, settle=True), 4)

    # the same step as one kernel over the per-parameter tensors
    ps = ddp.param_sync(plan, binds, rbind, c.order)
    t_ps = stream_ms(c, lambda: ps(c.stream), reps, warm=5, settle=True)
    chk = [torch.empty_like(t) for t in res]
    ddp.unflatten(plan, ddp.bind_params(plan, chk), c.out, stream=c.stream)   # out holds this sync
    torch.cuda.synchronize()
    same = all(torch.equal(x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32),
                           y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32))
               for x, y in zip(res, chk))
    out["param_sync"] = {
        "ms_per_step": round(t_ps, 4), "GBps": gbps(c.sync_bytes, t_ps),
        "speedup_vs_three_steps": round((tf + ts + tu) / t_ps, 2),
        "same_bits_as_three_steps": bool(same),
        "step": "every rank's per-parameter gradients averaged into per-parameter outputs "
                "in one launch (ddp_param_sync_run)"}
    out["carved_views"] = carved_view_rates(c, binds, reps, tu, t_ps)
    if wl.dtype == "f32":
        out["bf16"] = copy_rates_bf16(c, reps)
    log(f"copy path: {out}")
    return out


def leg_fused_sgd(c):
    """The average folded into a momentum-SGD step (ddp_sync_sgd_update)
    against the unfused sequence it replaces: the synchronisation, then the
    optimizer reading the averaged gradient back (torch's in-place ops); and
    the same step on per-parameter tensors."""
    torch, ddp, plan, wl, N, P = c.torch, c.ddp, c.plan, c.wl, c.N, c.P
    if c.args.no_fused_sgd:
        return None
    params = torch.empty(P, dtype=torch.float32, device=c.dev)
    c.W.device_normal_(params, 99, 7, 1.0)
    mbuf = torch.zeros(P, dtype=torch.float32, device=c.dev)
    lr, mu = 0.01, 0.9

    def fused_step():
        ddp.sync_sgd_update(plan, c.flats, params, lr, c.order, momentum_buf=mbuf, momentum=mu,
                            stream=c.stream)

    def unfused_step():
        c.sync()
        mbuf.mul_(mu).add_(c.out)
        params.add_(mbuf, alpha=-lr)

    t_f = stream_ms(c, fused_step, c.args.steps, warm=5)
    t_u = stream_ms(c, unfused_step, c.args.steps, warm=5)
    fb = N * P * wl.in_bytes + 4 * P * 4
    res = {"ms": round(t_f, 5), "GBps": gbps(fb, t_f), "bytes": fb, "unfused_ms": round(t_u, 5),
           "speedup_vs_unfused": round(t_u / t_f, 3),
           "step": f"momentum SGD (mu 0.9) on f32 parameters from {wl.dtype} gradients (the average "
                   f"as stored in {wl.out_dtype}); unfused = sync + torch mul_/add_"}
    # the same step on per-parameter tensors (gradients, parameters and
    # momentum buffers as autograd and the optimizer keep them)
    if N * P * wl.in_bytes <= (16 << 30):
        gviews = rank_grads(c)
        pp = [torch.empty(n, dtype=torch.float32, device=c.dev).normal_() for n in wl.numel]
        pm = [torch.zeros(n, dtype=torch.float32, device=c.dev) for n in wl.numel]
        step = ddp.param_sgd(plan, [ddp.bind_params(plan, g) for g in gviews],
                             ddp.bind_params(plan, pp), ddp.bind_params(plan, pm), None, c.order)
        t_p = stream_ms(c, lambda: step(lr, mu, c.stream), c.args.steps, warm=5)
        res["per_parameter"] = {
            "ms": round(t_p, 5), "GBps": gbps(fb, t_p),
            "step": "the same step on per-parameter gradients, parameters and momentum "
                    "(ddp_param_sgd_run)"}
    log(f"fused sgd: {res}")
    return res


def leg_overlap(c):
    """Syncs beside compute on a second stream.  First the two-bucket plan of
    the same tensors: DEEP_COMM averaged on an update stream while a GEMM
    (standing in for the first layer's backward) runs on a compute stream;
    exposed = overlapped time - compute time.  Then DDP's bucket-by-bucket
    schedule, flat and per-parameter.  Steps are timed back to back with both
    streams joined at every step boundary."""
    torch, ddp, plan, wl, P = c.torch, c.ddp, c.plan, c.wl, c.P
    if c.args.no_overlap or wl.name != "resnet50":
        return None
    tb = ddp.plan_two_bucket(wl.numel, wl.regions, wl.dtype)
    (dl, db, _, _), (fl_, _, _, _) = tb.bucket(0), tb.bucket(1)
    mat_a = torch.randn(4096, 4096, device=c.dev, dtype=torch.bfloat16)
    mat_b = torch.randn(4096, 4096, device=c.dev, dtype=torch.bfloat16)
    comp, upd, tried = side_by_side_streams(torch)

    def compute():
        with torch.cuda.stream(comp):
            torch.mm(mat_a, mat_b)

    def deep():
        # DEEP_COMM of the two-bucket plan (timing only: the cap plan's buffers
        # are read at the bucket's place), with that plan's occupancy policy
        ddp.sync_allreduce_avg_bucket(tb, 0, c.flats, c.out, c.order, stream=upd)

    def step_barrier():
        # a training step ends when both streams have: the next step's
        # backward needs the averaged gradients, and the next syncs the next
        # step's gradients
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

    def hidden(t_sync, t_alone, t_both):
        return {"exposed_sync_ms": round(max(t_both - t_alone, 0.0), 4),
                "hidden_fraction": round(1.0 - max(t_both - t_alone, 0.0) / t_sync, 3)}

    t_comp = timed([compute])
    res = {"plan": "two-bucket (DEEP_COMM %d, FIRST_COMM %d elements)" % (dl, fl_),
           "compute_ms": round(t_comp, 4),
           "compute": "bf16 GEMM 4096^3 on a second stream",
           "streams": ("side by side (hardware queues checked; %d tried)" % tried
                       if tried else "not found side by side: results are serial")}
    # under both occupancy policies, set on the plan (the process-wide policy
    # is not touched): the tuned cap reserves LDS that the GEMM's blocks would
    # need, "shared" leaves it free
    for policy in ("tuned", "shared"):
        tb.set_occupancy(policy)
        t_deep = timed([deep])
        t_both = timed([compute, deep])
        res[policy] = {"deep_sync_ms": round(t_deep, 4), "overlapped_ms": round(t_both, 4),
                       **hidden(t_deep, t_comp, t_both)}

    # The bucket-by-bucket schedule of DDP ([DDP] 3.2, [TR24] 十一): bucket b
    # (cap plan, last layers first) is averaged on the update stream as soon
    # as a stand-in for the backward of its layers -- a bf16 GEMM with FLOPs
    # in proportion to the bucket's share of the parameters, about 262 GFLOP
    # in all (ResNet-50's backward at 32 images per GPU) -- has finished on
    # the compute stream.
    buckets = [plan.bucket(b) for b in range(plan.n_buckets)]
    ks = [max(64, int(round(7808 * ln / P / 64)) * 64) for ln, _, _, _ in buckets]
    lhs = [torch.randn(4096, k, device=c.dev, dtype=torch.bfloat16) for k in ks]
    rhs = [torch.randn(k, 4096, device=c.dev, dtype=torch.bfloat16) for k in ks]
    ready = [torch.cuda.Event() for _ in buckets]
    # a plan object of its own for the overlapped syncs, so that its policy
    # is theirs alone
    sched_plan = ddp.plan_buckets(wl.numel, wl.bucket_cap_bytes, wl.dtype)

    def backward():
        with torch.cuda.stream(comp):
            for a, b, e in zip(lhs, rhs, ready):
                torch.mm(a, b)
                e.record(comp)

    def bucket_syncs(wait):
        for b in range(len(buckets)):
            if wait:
                upd.wait_event(ready[b])
            ddp.sync_allreduce_avg_bucket(sched_plan, b, c.flats, c.out, c.order, stream=upd)

    # the same schedule on per-parameter gradients (as autograd leaves them):
    # bucket b of one ddp_param_sync per step, run when ready
    pg = rank_grads(c)
    pout = [torch.empty(n, dtype=c.tout, device=c.dev) for n in wl.numel]
    pps = ddp.param_sync(plan, [ddp.bind_params(plan, g) for g in pg],
                         ddp.bind_params(plan, pout), c.order)

    def param_syncs(wait):
        for b in range(len(buckets)):
            if wait:
                upd.wait_event(ready[b])
            pps(upd, buckets=(b, 1))

    t_bwd = timed([backward])
    gflop = sum(2 * 4096 * k * 4096 for k in ks) / 1e9
    sched = {"buckets": len(buckets), "backward_gflop": round(gflop, 1),
             "backward_ms": round(t_bwd, 4)}
    per_param = {"sync": "ddp_param_sync_run_buckets, one bucket per launch"}
    sched["sync"] = "ddp_sync_allreduce_avg_bucket, one bucket per launch"
    for syncs, into, obj in ((bucket_syncs, sched, sched_plan), (param_syncs, per_param, pps)):
        for policy in ("tuned", "shared"):
            obj.set_occupancy(policy)
            t_syncs = timed([lambda: syncs(False)])
            t_sched = timed([backward, lambda: syncs(True)])
            into[policy] = {"syncs_ms": round(t_syncs, 4), "serial_ms": round(t_bwd + t_syncs, 4),
                            "overlapped_ms": round(t_sched, 4), **hidden(t_syncs, t_bwd, t_sched)}
    assert ddp.get_occupancy() == "tuned"
    sched["per_parameter"] = per_param
    res["schedule"] = sched
    log(f"overlap: {res}")
    return res


def leg_rank_sweep(c):
    """The same plan averaged over N = 2..32 virtual ranks (N > 16 takes the
    looped kernel): bandwidth against the number of concurrent streams."""
    torch, wl = c.torch, c.wl
    if c.args.no_rank_sweep or wl.name != "resnet50":
        return None
    pool = list(c.flats)
    for r in range(c.N, 32):
        t = torch.empty(c.P, dtype=c.tin, device=c.dev)
        c.W.device_normal_(t, r, wl.stream, wl.sigma)
        pool.append(t)
    sweep_out = torch.empty(c.P, dtype=c.tout, device=c.dev)
    res = {}
    for n in (2, 4, 6, 8, 9, 12, 16, 32):
        row = {}
        for o in ("ring", "seq"):
            call = c.ddp.make_sync(c.plan, pool[:n], sweep_out, o, stream=c.stream)
            ms = stream_ms(c, call, 50)
            row[o] = gbps((n * wl.in_bytes + wl.out_bytes) * c.P, ms)
        res[str(n)] = row
    log(f"rank sweep (GB/s): {res}")
    return res


def leg_in_place(c):
    """The all-reduce as the pages run it, in place (send buffer == receive
    buffer): the average overwrites rank 0's bucket buffer.  Runs after the
    parity leg because it rewrites rank 0's gradients."""
    res = {}
    for o in (() if c.args.no_in_place else ("ring", "seq")):
        call = c.ddp.make_sync(c.plan, c.flats, c.flats[0], o, stream=c.stream)
        ms = stream_ms(c, call, c.args.steps)
        res[o] = {"ms_per_sync": round(ms, 5), "GBps": gbps(c.sync_bytes, ms)}
    log(f"in place: {res}")
    return res or None


def leg_no_sync(c):
    """M micro-steps: with no_sync each rank accumulates locally (M - 1
    accumulates) and synchronises once; without it every micro-step also
    synchronises.  Separate buffers keep the benchmark's inputs untouched."""
    ddp, wl, N, P = c.ddp, c.wl, c.N, c.P
    if c.args.no_no_sync or 2 * N * P * wl.in_bytes > (16 << 30):
        return None
    M = 4
    local = [f.clone() for f in c.flats]
    micro = [f.clone() for f in c.flats]
    t_acc = stream_ms(c, lambda: ddp.accumulate(local, micro, stream=c.stream), c.args.steps)
    t_sync = stream_ms(c, lambda: ddp.sync_allreduce_avg(c.plan, local, c.out, c.order,
                                                         stream=c.stream), c.args.steps)
    res = {"micro_steps": M, "accumulate_ms": round(t_acc, 5),
           "accumulate_GBps": gbps(3 * N * P * wl.in_bytes, t_acc),
           "no_sync_ms": round((M - 1) * t_acc + t_sync, 5),
           "sync_every_step_ms": round((M - 1) * t_acc + M * t_sync, 5),
           "syncs_saved": M - 1}
    log(f"no_sync: {res}")
    return res


def latency(c, make_call, reps=2000):
    """Latency of a short synchronisation, in microseconds per call, three
    ways: `make_call(stream, prepared)` returns a zero-argument call that
    enqueues it on `stream` -- marshalling every argument per call
    (prepared=False) or once (prepared=True, one C call per step) -- and the
    prepared call captured into a HIP graph: one call per replay (the wall
    time of a replay), and 100 calls in one graph (device time per call)."""
    torch = c.torch

    def wall(fn, n):
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / n

    res = {"python_call_us": round(wall(make_call(c.stream, False), reps), 2),
           "prepared_call_us": round(wall(make_call(c.stream, True), reps), 2)}
    side = torch.cuda.Stream()
    side.wait_stream(c.stream)
    call = make_call(side, True)
    call()
    torch.cuda.synchronize()
    g1, g100 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1, stream=side):
        call()
    with torch.cuda.graph(g100, stream=side):
        for _ in range(100):
            call()
    torch.cuda.synchronize()
    res["graph_replay_us"] = round(wall(g1.replay, reps), 2)
    res["graph_of_100_us_per_call"] = round(wall(g100.replay, 20) / 100, 3)
    del g1, g100
    return res


def leg_noalloc(c):
    """The same synchronisation through ddp_sync_allreduce_avg_noalloc, which
    rebuilds the plan's ring tables in its static device buffer on every
    call (two small kernels before the reduce) instead of reading tables
    uploaded once: the cost of allocating nothing."""
    ddp = c.ddp
    if c.args.layout != "bucket-view" or c.order != "ring" or c.sync_bytes < (64 << 20):
        return None
    call = lambda: ddp.sync_allreduce_avg_noalloc(c.plan, c.flats, c.out, "ring",   # noqa: E731
                                                  stream=c.stream)
    ms = stream_ms(c, call, c.args.steps, warm=3, settle=True)
    res = {"ms_per_sync": round(ms, 5), "GBps": gbps(c.sync_bytes, ms),
           "vs_prepared_tables": round(c.kern_ms / ms, 4),
           "call": "ddp_sync_allreduce_avg_noalloc, K back-to-back calls between one event pair"}
    log(f"no-allocation sync: {res}")
    return res


def leg_tiny_latency(c):
    """The latency-bound workload (tiny: 15 KB per sync): its sync through
    the plain Python call, the prepared call and graph replay."""
    ddp = c.ddp
    if c.wl.name != "tiny":
        return None

    def make_call(st, prepared):
        if prepared:
            return ddp.make_sync(c.plan, c.flats, c.out, c.order, stream=st)
        return lambda: ddp.sync_allreduce_avg(c.plan, c.flats, c.out, c.order, stream=st)

    res = latency(c, make_call)
    log(f"tiny latency: {res}")
    return res


def leg_small_means(c):
    """The same mean all-reduce at its other call sites ([TR24] 十二, 十三):
    the BN running statistics -- every BN layer's running mean and running
    variance, one contiguous range of 2 x (BN channels) f32 values -- and a
    validation record of 3 scalars (loss, top-1, top-5), over the N virtual
    ranks, ring order; checked against the oracle and timed as latency."""
    import oracle
    torch, ddp, wl, N, np = c.torch, c.ddp, c.wl, c.N, c.np
    if wl.name != "resnet50":
        return None
    bn_channels = sum(p.numel for p in wl.params if p.region == c.W.REGION_BN_WEIGHT)
    res = {}
    rng = np.random.default_rng(12)
    for name, length in (("bn_running_stats", 2 * bn_channels), ("metric_record", 3)):
        xs = [(rng.standard_normal(length) * 0.5 + 1.0).astype(np.float32) for _ in range(N)]
        ins = [torch.from_numpy(x).to(c.dev) for x in xs]
        out = torch.empty(length, device=c.dev)
        plan = ddp.plan_buckets([length], 1 << 40, "f32")

        def make_call(st, prepared, plan=plan, ins=ins, out=out):
            if prepared:
                return ddp.make_sync(plan, ins, out, c.order, stream=st)
            return lambda: ddp.bucket_allreduce_avg(ins, out, c.order, stream=st)

        lat = latency(c, make_call, reps=1000)
        ddp.bucket_allreduce_avg(ins, out, c.order, stream=c.stream)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        want = oracle.bucket_avg(xs, c.order)
        lat["elements"] = length
        lat["parity"] = ("bitwise equal to the CPU oracle"
                         if np.array_equal(got.view(np.uint32), want.view(np.uint32)) else
                         "MISMATCH against the CPU oracle")
        res[name] = lat
    log(f"small means: {res}")
    return res


def calibrate(torch):
    """A plain 1 GiB device-to-device copy, 10 times: the kernel of known size
    that scales the FETCH_SIZE / WRITE_SIZE counters."""
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": a.numel() * 4, "copies": 10}), flush=True)


def dtype_label(wl):
    """The arithmetic the path computes in: the FP32 fold, with the input and
    output element types when they are not f32."""
    if wl.dtype == wl.out_dtype == "f32":
        return "f32"
    return f"{wl.dtype}->{wl.out_dtype} (f32 accumulate)"


def measure(args, cpu_seconds):
    """One workload measured in this process: its JSON record (the line a
    child prints)."""
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    c = setup(args)
    sensors_before = hwmon_readings(torch)
    timed_steps(c)
    sensors_after = hwmon_readings(torch)
    per_param = args.layout == "per-parameter"
    extras = (args.extras == "on") if args.extras else c.wl.name == "resnet50"
    copy_only = args.extras is None and c.wl.name == "many_small"   # the copies of many tensors
    sgd_only = args.extras is None and c.wl.name == "llama7b"       # the fused step on bf16 gradients
    cold = leg_cold_mall(c)
    ceiling = None if per_param else leg_ceiling(c)
    other = leg_other_orders(c)
    if per_param:
        parity, cpu = leg_parity_per_parameter(c), None
    else:
        parity, cpu = leg_parity_and_cpu(c, cpu_seconds)
    more = {}
    if extras and not per_param:
        more = {"per_bucket": leg_per_bucket(c), "copy_path": leg_copy_path(c),
                "fused_sgd": leg_fused_sgd(c), "overlap": leg_overlap(c),
                "rank_sweep_GBps": leg_rank_sweep(c), "in_place": leg_in_place(c),
                "no_sync": leg_no_sync(c), "small_means": leg_small_means(c)}
    elif copy_only and not per_param:
        more = {"copy_path": leg_copy_path(c)}
    elif sgd_only and not per_param:
        more = {"fused_sgd": leg_fused_sgd(c)}
    tiny = leg_tiny_latency(c)
    noalloc = leg_noalloc(c)

    wl, P, np = c.wl, c.P, c.np
    kernel = "params_fast" if per_param else "reduce_fast"
    traffic, traffic_source = measured_traffic(wl.name, c.order, args.layout)
    record = {
        "metric": METRIC,
        "value": round(c.value, 1),
        "unit": "GB/s",
        "pct_of_peak": round(100.0 * c.value / HBM_PEAK_GBPS, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(c.ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label(wl),
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {len(wl.params)} gradient tensors, "
                               f"{P} elements, {c.N} virtual ranks, {c.plan.n_buckets} buckets",
                   "virtual_ranks": c.N, "elements": P, "buckets": c.plan.n_buckets,
                   "bucket_cap_bytes": wl.bucket_cap_bytes,
                   "plan": "two-bucket" if wl.two_bucket else "cap",
                   "order": c.order, "grad_dtype": wl.dtype, "out_dtype": wl.out_dtype,
                   "grad_layout": ("per-parameter tensors of every rank, read where they lie by one "
                                   "kernel (ddp_param_sync_run)" if per_param else
                                   "bucket view (gradients live in the per-rank flat buckets)"),
                   "bytes_per_sync": c.sync_bytes,
                   "device": torch.cuda.get_device_name(0)},
        "roofline": {"bound": "hbm", "achieved": round(c.achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(c.achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "traffic_source": traffic_source,
                     "kernel": kernel + " (one launch per sync)",
                     "kernel_ms": round(c.kern_ms, 5),
                     "kernel_ms_source": "event pair around the K timed launches on the launch "
                                         "stream, / K",
                     "single_launch_ms_median": round(float(np.median(c.launch_ms)), 5),
                     "single_launch_ms_min": round(min(c.launch_ms), 5)},
        "ramp": c.ramp,
        "cold_mall": cold,
        "ceiling": ceiling,
        "cpu_baseline": cpu,
        "parity": parity,
        "other_orders": other,
        **({"latency": tiny} if tiny else {}),
        **({"noalloc": noalloc} if noalloc else {}),
        **{k: v for k, v in more.items() if v is not None},
        "env": dict(run_environment(torch),
                    sensors={"before_timed_steps": sensors_before,
                             "after_timed_steps": sensors_after}),
    }
    return record


# keys every record repeats; a workload under "configs" drops them
_SHARED_KEYS = ("metric", "unit", "n_gpus", "steps", "warmup", "higher_is_better", "scaling",
                "vs_baseline", "data")


def run_child(args, workload, cpu_seconds, headline, layout=None):
    """Measures one workload in a fresh child process (started by this
    process, which has not touched the GPU) and returns its record."""
    cmd = [sys.executable, "-u", os.path.abspath(__file__), "--child", "--workload", workload,
           "--steps", str(args.steps), "--warmup", str(args.warmup),
           "--ramp-ms", str(args.ramp_ms), "--cpu-seconds", str(cpu_seconds)]
    for flag in ("cpu_baseline", "copy_path", "ceiling", "fused_sgd", "overlap", "no_sync",
                 "in_place", "rank_sweep", "cold", "per_bucket"):
        if getattr(args, "no_" + flag):
            cmd.append("--no-" + flag.replace("_", "-"))
    if args.extras:
        cmd += ["--extras", args.extras]
    if headline:
        cmd += ["--layout", args.layout] + (["--order", args.order] if args.order else [])
    elif layout:
        cmd += ["--layout", layout]
    log(f"bench: {workload} ({layout or 'bucket-view'}) in a child process")
    t0 = time.perf_counter()
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
    lines = [l for l in proc.stdout.splitlines() if l.startswith("{")]
    if proc.returncode != 0 or not lines:
        return {"error": f"child exited with status {proc.returncode}"}
    rec = json.loads(lines[-1])
    rec["child_wall_s"] = round(time.perf_counter() - t0, 1)
    return rec


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the N virtual ranks of a synchronisation live in that GPU's HBM", file=sys.stderr)
        sys.exit(2)
    if args.calibrate:
        import torch
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        calibrate(torch)
        return
    if args.child:
        print(json.dumps(measure(args, args.cpu_seconds)), flush=True)
        return

    # Parent: never touches the GPU; every workload runs in a child of its own.
    if args.settle_seconds > 0:
        log(f"bench: idle {args.settle_seconds:.0f} s before the first GPU call")
        time.sleep(args.settle_seconds)
    line = run_child(args, args.workload, args.cpu_seconds, headline=True)
    if "error" in line:
        log(f"bench: the headline workload {args.workload} failed: {line['error']}")
        sys.exit(1)
    names = [w for w in args.configs.split(",") if w and w != "none" and w != args.workload]
    configs = {}
    for w in names:
        if args.config_settle_seconds > 0:
            time.sleep(args.config_settle_seconds)
        name, _, layout = w.partition(":")
        rec = run_child(args, name, args.config_cpu_seconds, headline=False, layout=layout or None)
        configs[w] = {k: v for k, v in rec.items() if k not in _SHARED_KEYS}
    line["configs"] = configs
    line["protocol"] = {
        "processes": "each workload in a fresh child process; the parent never touches the GPU",
        "settle_seconds_before_first": args.settle_seconds,
        "settle_seconds_between": args.config_settle_seconds,
        "order": [args.workload] + names,
        "per_workload": f"ramp >= {args.ramp_ms:.0f} ms of back-to-back syncs (the first "
                        f"{args.steps} timed: ramp.without_ramp), {args.warmup} warm-up syncs, "
                        f"{args.steps} timed syncs; then the flushed-MALL leg, the probe, the "
                        f"other order, parity and the CPU oracle"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
