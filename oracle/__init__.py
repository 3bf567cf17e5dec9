"""CPU ORACLE -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU statement of bucketed gradient all-reduce
averaging, used to check the HIP library.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it.  It shares no code with ``gradient_allreduce_averaging_amd`` and
imports nothing from it; inputs come from ``workloads`` (seeded generators
with none of the method's arithmetic) or are passed in by the caller.

Pages cited (title, section):
  [DDP]  "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel)
  [TR24] "(24) NCCL通信与分布式数据并行" (tech-renaissance.cn)
  [TR16] "(16) DTensor：一张图纸，多卡共享的分布式张量抽象" (tech-renaissance.cn)
  [DL]   "DDP分布式训练–数据加载和训练NCCL" (139.9.1.231)

Readings taken where the pages leave a step open (each is listed in the
design notes with its alternative):
  * bucket cap: "25MB" is 25 MiB, counted in bytes of the gradient dtype; a
    bucket closes *before* it would exceed the cap; a lone parameter larger
    than the cap gets a bucket of its own.
  * ring chunks: contiguous chunks of C = ceil(L/N) elements per bucket, the
    last one short or empty (the ceil split of [DL] section 3, custom sampler).
  * ring start: chunk c starts accumulating at rank (c+1) mod N ([DDP]
    section 2.11 round formula with rounds counted from 1).  The simulator
    also supports start offset 0, the convention of the printed tables.
  * scale: multiply by fl(1/N) ([TR24] section 九), applied to the FP32 sum.
  * two-bucket plan: bucket 0 = DEEP_COMM (the DEEP region), bucket 1 =
    FIRST_COMM (BN_BIAS, BN_WEIGHT, FC_BIAS, FC_WEIGHT, FIRST in region
    order), parameters in registration order inside a region ([TR24]
    sections 七/八; region layout of [TR16] section 四); an empty bucket is
    dropped.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
what the pages or mathematics fix (printed worked example, closed forms,
exact rational sums, brute force, IEEE special cases).  Unpinned by the
pages and defined only by the readings above: the bucket cap rule, the
chunk rule, the ring start rank 1, and the scale for N not a power of two.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import List, Sequence

import numpy as np

SEQ = "seq"
RING = "ring"
_ORDER_CODE = {SEQ: 0, RING: 1}
_DTYPE_CODE = {"f32": 0, "bf16": 1}
_NP_DTYPE = {"f32": np.float32, "bf16": np.uint16}   # bf16 held as bit patterns

# Region tags of the two-bucket split, in memory (enum) order ([TR24] section 七).
BN_BIAS, BN_WEIGHT, FC_BIAS, FC_WEIGHT, FIRST, DEEP = range(6)
FIRST_COMM_REGIONS = (BN_BIAS, BN_WEIGHT, FC_BIAS, FC_WEIGHT, FIRST)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_core.c")
_LIB = os.path.join(_HERE, "liboracle_core.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C core with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared",
                               "-ffp-contract=off", "-fno-fast-math", "-Wall",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def load_core(path: str):
    """Load a compiled oracle core and declare its C signatures."""
    lib = ctypes.CDLL(path)
    lib.oracle_rne_bf16.restype = ctypes.c_uint16
    lib.oracle_rne_bf16.argtypes = [ctypes.c_float]
    lib.oracle_rne_bf16_array.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_bucket_avg.restype = ctypes.c_int
    lib.oracle_bucket_avg.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p]
    lib.oracle_bucket_range_avg.restype = ctypes.c_int
    lib.oracle_bucket_range_avg.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p]
    lib.oracle_sampled_avg.restype = ctypes.c_int
    lib.oracle_sampled_avg.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.oracle_sgd_step.restype = ctypes.c_int
    lib.oracle_sgd_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_int64, ctypes.c_float, ctypes.c_float]
    lib.oracle_accumulate.restype = ctypes.c_int
    lib.oracle_accumulate.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64]
    return lib


def _core():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = load_core(_LIB)
    return _lib


# ---------------------------------------------------------------------------
# Bucket plans
# ---------------------------------------------------------------------------

@dataclass
class Plan:
    """A bucket plan.  ``buckets[b]`` lists parameter indices in their order
    inside bucket b; buckets sit back to back in the flat gradient buffer."""
    numel: List[int]
    buckets: List[List[int]]

    @property
    def n_buckets(self) -> int:
        return len(self.buckets)

    @property
    def bucket_len(self) -> List[int]:
        return [sum(self.numel[p] for p in b) for b in self.buckets]

    @property
    def bucket_base(self) -> List[int]:
        base, out = 0, []
        for ln in self.bucket_len:
            out.append(base)
            base += ln
        return out

    @property
    def total(self) -> int:
        return sum(self.numel)

    def param_location(self):
        """(bucket, offset within bucket) of every parameter."""
        loc = [None] * len(self.numel)
        for b, ps in enumerate(self.buckets):
            off = 0
            for p in ps:
                loc[p] = (b, off)
                off += self.numel[p]
        return loc


def plan_cap(numel: Sequence[int], bucket_cap_bytes: int, elem_bytes: int) -> Plan:
    """Greedy packing in reverse registration order ([DDP] section 4.2:
    parameters reversed, then buckets of bucket_size_mb; [DDP] section 3.2:
    the last layer lands in the first bucket).  A bucket closes before the
    next parameter would push it past the cap."""
    if bucket_cap_bytes <= 0 or elem_bytes <= 0 or any(n < 0 for n in numel):
        raise ValueError("invalid plan arguments")
    buckets, cur, cur_bytes = [], [], 0
    for p in reversed(range(len(numel))):
        nb = numel[p] * elem_bytes
        if cur and cur_bytes + nb > bucket_cap_bytes:
            buckets.append(cur)
            cur, cur_bytes = [], 0
        cur.append(p)
        cur_bytes += nb
    if cur:
        buckets.append(cur)
    return Plan(list(numel), buckets)


def plan_two_bucket(numel: Sequence[int], region: Sequence[int]) -> Plan:
    """DEEP_COMM then FIRST_COMM ([TR24] section 八).  FIRST_COMM is the
    contiguous region span BN_BIAS..FIRST; inside a region parameters keep
    registration order (the memory plan walks regions in enum order and
    places tensors one after another, [TR16] section 四)."""
    if len(numel) != len(region) or any(n < 0 for n in numel):
        raise ValueError("invalid plan arguments")
    if any(r not in FIRST_COMM_REGIONS and r != DEEP for r in region):
        raise ValueError("unknown region tag")
    deep = [p for p in range(len(numel)) if region[p] == DEEP]
    first = [p for reg in FIRST_COMM_REGIONS for p in range(len(numel)) if region[p] == reg]
    return Plan(list(numel), [b for b in (deep, first) if b])


# ---------------------------------------------------------------------------
# Reduce + scale
# ---------------------------------------------------------------------------

def _ptrs(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def bucket_avg(xs: Sequence[np.ndarray], order: str, in_dtype: str = "f32",
               out_dtype: str = None) -> np.ndarray:
    """Average one bucket held by len(xs) ranks (see oracle_core.c)."""
    out_dtype = out_dtype or in_dtype
    xs = [np.ascontiguousarray(x, dtype=_NP_DTYPE[in_dtype]) for x in xs]
    L = xs[0].size
    if any(x.size != L for x in xs):
        raise ValueError("rank buffers differ in length")
    out = np.empty(L, dtype=_NP_DTYPE[out_dtype])
    rc = _core().oracle_bucket_avg(_ptrs(xs), len(xs), L, _ORDER_CODE[order],
                                   _DTYPE_CODE[in_dtype], _DTYPE_CODE[out_dtype],
                                   out.ctypes.data)
    if rc:
        raise ValueError("oracle rejected the arguments")
    return out


def bucket_range_avg(xs: Sequence[np.ndarray], bucket_len: int, lo: int, order: str,
                     in_dtype: str = "f32", out_dtype: str = None,
                     out: np.ndarray = None) -> np.ndarray:
    """Elements [lo, lo + n) of one bucket's average, n = xs[r].size: xs[r]
    holds rank r's elements lo..lo+n-1 of a bucket of bucket_len elements.
    Each element is folded as by bucket_avg at its position in the whole
    bucket.  The C call releases the GIL, so pieces can run on threads."""
    out_dtype = out_dtype or in_dtype
    xs = [np.ascontiguousarray(x, dtype=_NP_DTYPE[in_dtype]) for x in xs]
    n = xs[0].size
    if any(x.size != n for x in xs):
        raise ValueError("rank pieces differ in length")
    if out is None:
        out = np.empty(n, dtype=_NP_DTYPE[out_dtype])
    elif out.dtype != _NP_DTYPE[out_dtype] or out.size != n or not out.flags.c_contiguous:
        raise ValueError("out does not match the piece")
    rc = _core().oracle_bucket_range_avg(_ptrs(xs), len(xs), bucket_len, lo, n,
                                         _ORDER_CODE[order], _DTYPE_CODE[in_dtype],
                                         _DTYPE_CODE[out_dtype], out.ctypes.data)
    if rc:
        raise ValueError("oracle rejected the arguments")
    return out


def sync_avg(plan: Plan, rank_flats: Sequence[np.ndarray], order: str,
             in_dtype: str = "f32", out_dtype: str = None) -> np.ndarray:
    """One whole synchronisation: every bucket averaged on its own, since each
    bucket is its own all-reduce ([DDP] section 4.2; [TR24] section 九)."""
    out_dtype = out_dtype or in_dtype
    out = np.empty(plan.total, dtype=_NP_DTYPE[out_dtype])
    for base, ln in zip(plan.bucket_base, plan.bucket_len):
        out[base:base + ln] = bucket_avg([f[base:base + ln] for f in rank_flats],
                                         order, in_dtype, out_dtype)
    return out


def sampled_avg(vals: np.ndarray, pos: np.ndarray, lens: np.ndarray, order: str,
                in_dtype: str = "f32", out_dtype: str = None) -> np.ndarray:
    """Average S single elements: vals[s, r] is rank r's value of sample s,
    pos[s] its position inside its bucket, lens[s] the bucket length."""
    out_dtype = out_dtype or in_dtype
    vals = np.ascontiguousarray(vals, dtype=_NP_DTYPE[in_dtype])
    S, N = vals.shape
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int64)
    out = np.empty(S, dtype=_NP_DTYPE[out_dtype])
    rc = _core().oracle_sampled_avg(vals.ctypes.data, pos.ctypes.data, lens.ctypes.data,
                                    S, N, _ORDER_CODE[order], _DTYPE_CODE[in_dtype],
                                    _DTYPE_CODE[out_dtype], out.ctypes.data)
    if rc:
        raise ValueError("oracle rejected the arguments")
    return out


def rne_bf16(y: np.ndarray) -> np.ndarray:
    """f32 -> bf16 bit patterns, round to nearest, ties to even."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.size, dtype=np.uint16)
    _core().oracle_rne_bf16_array(y.ctypes.data, y.size, out.ctypes.data)
    return out.reshape(y.shape)


def sgd_step(param: np.ndarray, grad: np.ndarray, lr: float, grad_dtype: str = "f32",
             momentum_buf: np.ndarray = None, momentum: float = 0.0):
    """One SGD step in place on float32 ``param`` (and ``momentum_buf``):
    theta <- theta - lr * g ([DDP] section 5.3), g the averaged gradient as
    stored; with a momentum buffer v = mu * v + g first (see oracle_core.c)."""
    assert param.dtype == np.float32 and param.flags.c_contiguous
    g = np.ascontiguousarray(grad, dtype=_NP_DTYPE[grad_dtype])
    if g.size != param.size:
        raise ValueError("gradient and parameter sizes differ")
    mptr = None
    if momentum_buf is not None:
        assert momentum_buf.dtype == np.float32 and momentum_buf.flags.c_contiguous
        mptr = momentum_buf.ctypes.data
    rc = _core().oracle_sgd_step(param.ctypes.data, mptr, g.ctypes.data, _DTYPE_CODE[grad_dtype],
                                 param.size, np.float32(lr), np.float32(momentum))
    if rc:
        raise ValueError("oracle rejected the arguments")


def sync_sgd(plan: Plan, rank_flats: Sequence[np.ndarray], order: str, param: np.ndarray,
             lr: float, in_dtype: str = "f32", out_dtype: str = None,
             momentum_buf: np.ndarray = None, momentum: float = 0.0) -> np.ndarray:
    """The synchronisation followed by one SGD step on the flat parameters
    (updated in place); returns the averaged gradient."""
    out_dtype = out_dtype or in_dtype
    avg = sync_avg(plan, rank_flats, order, in_dtype, out_dtype)
    sgd_step(param, avg, lr, out_dtype, momentum_buf, momentum)
    return avg


def accumulate(dst: np.ndarray, src: np.ndarray, dtype: str = "f32"):
    """dst += src in place: the local gradient accumulation of no_sync
    micro-steps ([DDP] section 5.2)."""
    assert dst.dtype == _NP_DTYPE[dtype] and dst.flags.c_contiguous
    s = np.ascontiguousarray(src, dtype=_NP_DTYPE[dtype])
    if s.size != dst.size:
        raise ValueError("sizes differ")
    if _core().oracle_accumulate(dst.ctypes.data, s.ctypes.data, _DTYPE_CODE[dtype], dst.size):
        raise ValueError("oracle rejected the arguments")


def no_sync_then_sync(plan: Plan, micro: Sequence[Sequence[np.ndarray]], order: str,
                      dtype: str = "f32") -> np.ndarray:
    """micro[m][r]: rank r's flat gradient of micro-step m.  Gradients are
    accumulated per rank in micro-step order (no synchronisation), then the
    accumulated buffers are synchronised once."""
    local = [np.array(micro[0][r], copy=True) for r in range(len(micro[0]))]
    for m in range(1, len(micro)):
        for r in range(len(local)):
            accumulate(local[r], micro[m][r], dtype)
    return sync_avg(plan, local, order, dtype, dtype)


# ---------------------------------------------------------------------------
# Flatten / unflatten: bit copies through the plan offsets ([DDP] section 4.2,
# bucket.flat_grad built from the parameters' gradients and viewed back).
# ---------------------------------------------------------------------------

def flatten(plan: Plan, grads: Sequence[np.ndarray]) -> np.ndarray:
    flat = np.empty(plan.total, dtype=grads[0].dtype)
    for b, base in zip(plan.buckets, plan.bucket_base):
        off = base
        for p in b:
            flat[off:off + plan.numel[p]] = grads[p].reshape(-1)
            off += plan.numel[p]
    return flat


def unflatten(plan: Plan, flat: np.ndarray) -> List[np.ndarray]:
    out = [None] * len(plan.numel)
    for b, base in zip(plan.buckets, plan.bucket_base):
        off = base
        for p in b:
            out[p] = flat[off:off + plan.numel[p]].copy()
            off += plan.numel[p]
    return out


# ---------------------------------------------------------------------------
# Literal ring all-reduce simulator ([DDP] sections 2.10-2.12): N ranks, each
# holding its own buffer, exchanging chunks round by round.  Small cases only.
# ---------------------------------------------------------------------------

def ring_chunks(L: int, N: int):
    C = -(-L // N) if L else 0
    return [(min(k * C, L), min((k + 1) * C, L)) for k in range(N)]


def ring_allreduce(bufs: Sequence[np.ndarray], s0: int = 1, trace: bool = False):
    """Run reduce-scatter then all-gather on copies of ``bufs`` (float32).

    Ring 0 -> 1 -> ... -> N-1 -> 0.  Reduce-scatter round t (t = 0..N-2):
    rank i sends chunk (i - s0 - t) mod N to rank i+1, which stores
    received + own.  All-gather round t: rank i forwards chunk
    (i + 1 - s0 - t) mod N (its newest complete chunk) to rank i+1, which
    overwrites its copy.  With s0 = 0 this is the walk-through as printed;
    with s0 = 1 it is the round formula with rounds counted from 1.

    Returns a dict with the final buffers (sums, not yet scaled), the
    per-round snapshots when ``trace`` is set, the rounds run and the
    elements each rank sent.
    """
    N = len(bufs)
    b = [np.array(x, dtype=np.float32, copy=True) for x in bufs]
    L = b[0].size
    ch = ring_chunks(L, N)
    sent = [0] * N
    rs_snap, ag_snap = [], []
    rounds = 0
    for t in range(N - 1):
        msgs = []
        for i in range(N):
            c = (i - s0 - t) % N
            lo, hi = ch[c]
            msgs.append(((i + 1) % N, c, b[i][lo:hi].copy()))
            sent[i] += hi - lo
        for dst, c, data in msgs:
            lo, hi = ch[c]
            b[dst][lo:hi] = data + b[dst][lo:hi]
        rounds += 1
        if trace:
            rs_snap.append([x.copy() for x in b])
    owner_chunk = [(i + 1 - s0) % N for i in range(N)]
    for t in range(N - 1):
        msgs = []
        for i in range(N):
            c = (i + 1 - s0 - t) % N
            lo, hi = ch[c]
            msgs.append(((i + 1) % N, c, b[i][lo:hi].copy()))
            sent[i] += hi - lo
        for dst, c, data in msgs:
            lo, hi = ch[c]
            b[dst][lo:hi] = data
        rounds += 1
        if trace:
            ag_snap.append([x.copy() for x in b])
    return {"final": b, "rs": rs_snap, "ag": ag_snap, "rounds": rounds,
            "sent": sent, "owner_chunk": owner_chunk, "chunks": ch}


def ring_allreduce_avg(bufs: Sequence[np.ndarray], s0: int = 1) -> List[np.ndarray]:
    """Simulated ring all-reduce followed by the per-rank 1/N scale."""
    N = len(bufs)
    if N == 1:
        return [np.array(bufs[0], dtype=np.float32, copy=True)]
    inv = np.float32(1.0) / np.float32(N)
    return [(x * inv).astype(np.float32) for x in ring_allreduce(bufs, s0)["final"]]
