"""Python binding of libddp.so: bucketed gradient synchronisation on MI355X.

Argument marshalling only -- every step runs in the HIP library through its
C ABI (``include/ddp.h``).  PyTorch supplies device memory and streams:
tensors are passed by ``data_ptr()``, streams by ``torch.cuda.Stream``
handles.  Importing this module loads ``libddp.so`` and raises if it has not
been built; there is no fallback implementation.

Names follow the C ABI: ``plan_buckets``, ``plan_two_bucket``,
``bind_params``, ``flatten``, ``bucket_allreduce_avg``,
``sync_allreduce_avg``, ``sync_sgd_update``, ``accumulate``, ``unflatten``;
``make_sync`` resolves a synchronisation once for repeated calls.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libddp.so")

SEQUENTIAL = 0
RING = 1
_ORDERS = {"seq": SEQUENTIAL, "sequential": SEQUENTIAL, "ring": RING,
           SEQUENTIAL: SEQUENTIAL, RING: RING}
F32 = 0
BF16 = 1
_DTYPES = {"f32": F32, "float32": F32, "bf16": BF16, "bfloat16": BF16, F32: F32, BF16: BF16}

REGION_BN_BIAS, REGION_BN_WEIGHT, REGION_FC_BIAS, REGION_FC_WEIGHT, REGION_FIRST, REGION_DEEP = range(6)

STATUS = {0: "DDP_OK", 1: "DDP_ERR_INVALID_ARG", 2: "DDP_ERR_UNSUPPORTED", 3: "DDP_ERR_OVERFLOW",
          4: "DDP_ERR_ALIAS", 5: "DDP_ERR_HIP", 6: "DDP_ERR_NOMEM", 7: "DDP_ERR_CAPACITY"}


class DDPError(RuntimeError):
    def __init__(self, status: int, call: str, detail: str = ""):
        self.status = status
        msg = f"{call} failed: {STATUS.get(status, status)}"
        super().__init__(msg + (f" ({detail})" if detail else ""))


def _hip_runtimes_mapped():
    try:
        with open("/proc/self/maps") as f:
            return {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return set()


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950)")
    # torch owns the device memory and streams handed to the library, so the
    # library must run on torch's HIP runtime: load torch first, and the
    # libamdhip64.so.7 dependency of libddp.so then resolves to the runtime
    # torch already mapped instead of a second copy from /opt/rocm.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded in this process "
                          f"({sorted(runtimes)}); import torch before libddp.so")
    c_i64p = ctypes.POINTER(ctypes.c_int64)
    c_i32p = ctypes.POINTER(ctypes.c_int32)
    vp = ctypes.c_void_p
    sig = {
        "ddp_plan_buckets": ([c_i64p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int,
                              ctypes.POINTER(vp)], ctypes.c_int),
        "ddp_plan_two_bucket": ([c_i64p, ctypes.POINTER(ctypes.c_uint8), ctypes.c_int32,
                                 ctypes.c_int, ctypes.POINTER(vp)], ctypes.c_int),
        "ddp_plan_free": ([vp], None),
        "ddp_plan_num_buckets": ([vp], ctypes.c_int32),
        "ddp_plan_total": ([vp], ctypes.c_int64),
        "ddp_plan_bucket": ([vp, ctypes.c_int32, c_i64p, c_i64p, c_i32p, c_i32p], ctypes.c_int),
        "ddp_plan_slot_param": ([vp, ctypes.c_int32, c_i32p], ctypes.c_int),
        "ddp_plan_param": ([vp, ctypes.c_int32, c_i32p, c_i64p], ctypes.c_int),
        "ddp_plan_prepare": ([vp], ctypes.c_int),
        "ddp_plan_prepare_ranks": ([vp, ctypes.c_int32], ctypes.c_int),
        "ddp_set_occupancy": ([ctypes.c_int], ctypes.c_int),
        "ddp_get_occupancy": ([], ctypes.c_int),
        "ddp_plan_set_occupancy": ([vp, ctypes.c_int], ctypes.c_int),
        "ddp_plan_get_occupancy": ([vp], ctypes.c_int),
        "ddp_param_sync_set_occupancy": ([vp, ctypes.c_int], ctypes.c_int),
        "ddp_param_sync_get_occupancy": ([vp], ctypes.c_int),
        "ddp_sync_allreduce_avg_bucket": ([vp, ctypes.c_int32, ctypes.POINTER(vp), ctypes.c_int32,
                                           ctypes.c_int, ctypes.c_int, vp, vp], ctypes.c_int),
        "ddp_bind_params": ([vp, ctypes.POINTER(vp), vp, ctypes.POINTER(vp)], ctypes.c_int),
        "ddp_binding_free": ([vp], None),
        "ddp_flatten": ([vp, vp, ctypes.c_int32, vp, ctypes.c_int, vp], ctypes.c_int),
        "ddp_unflatten": ([vp, vp, ctypes.c_int32, vp, ctypes.c_int, vp], ctypes.c_int),
        "ddp_bucket_allreduce_avg": ([ctypes.POINTER(vp), ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp],
                                     ctypes.c_int),
        "ddp_sync_allreduce_avg": ([vp, ctypes.POINTER(vp), ctypes.c_int32, ctypes.c_int,
                                    ctypes.c_int, vp, vp], ctypes.c_int),
        "ddp_sync_allreduce_avg_noalloc": ([vp, ctypes.POINTER(vp), ctypes.c_int32, ctypes.c_int,
                                            ctypes.c_int, vp, vp], ctypes.c_int),
        "ddp_sync_sgd_update": ([vp, ctypes.POINTER(vp), ctypes.c_int32, ctypes.c_int, ctypes.c_int,
                                 vp, vp, vp, ctypes.c_float, ctypes.c_float, vp], ctypes.c_int),
        "ddp_param_sync_create": ([vp, ctypes.POINTER(vp), ctypes.c_int32, vp, ctypes.c_int,
                                   ctypes.c_int, ctypes.POINTER(vp)], ctypes.c_int),
        "ddp_param_sync_run": ([vp, vp], ctypes.c_int),
        "ddp_param_sync_free": ([vp], None),
        "ddp_param_sgd_create": ([vp, ctypes.POINTER(vp), ctypes.c_int32, vp, vp, vp, ctypes.c_int,
                                  ctypes.c_int, ctypes.POINTER(vp)], ctypes.c_int),
        "ddp_param_sgd_run": ([vp, ctypes.c_float, ctypes.c_float, vp], ctypes.c_int),
        "ddp_param_sync_run_buckets": ([vp, ctypes.c_int32, ctypes.c_int32, vp], ctypes.c_int),
        "ddp_param_sgd_run_buckets": ([vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                       ctypes.c_float, vp], ctypes.c_int),
        "ddp_accumulate": ([ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int32, ctypes.c_int64,
                            ctypes.c_int, vp], ctypes.c_int),
        "ddp_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "ddp_abi_version": ([], ctypes.c_int32),
        "ddp_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def _check(status: int, call: str):
    if status != 0:
        detail = lib.ddp_last_error().decode() if status == 5 else ""
        raise DDPError(status, call, detail)


def _ptr_array(ptrs: Sequence[int]):
    return (ctypes.c_void_p * len(ptrs))(*[ctypes.c_void_p(int(p)) for p in ptrs])


# ---------------------------------------------------------------- torch glue

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported gradient dtype {t.dtype}")


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev_ptr(t) -> int:
    if not t.is_cuda:
        raise ValueError("tensor is not on a GPU")
    if not t.is_contiguous():
        raise ValueError("tensor is not contiguous")
    return t.data_ptr()


# ---------------------------------------------------------------- plans

class Plan:
    """Owner of a ``ddp_plan_t``."""

    def __init__(self, handle: ctypes.c_void_p, dtype: int, numel: Sequence[int]):
        self._h = handle
        self.dtype = dtype
        self.numel = [int(n) for n in numel]

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and lib is not None:
            lib.ddp_plan_free(h)

    @property
    def n_buckets(self) -> int:
        return lib.ddp_plan_num_buckets(self._h)

    @property
    def total(self) -> int:
        return lib.ddp_plan_total(self._h)

    def bucket(self, b: int):
        """(len, base, first_slot, n_slots) of bucket b."""
        ln, base = ctypes.c_int64(), ctypes.c_int64()
        fs, ns = ctypes.c_int32(), ctypes.c_int32()
        _check(lib.ddp_plan_bucket(self._h, b, ctypes.byref(ln), ctypes.byref(base),
                                   ctypes.byref(fs), ctypes.byref(ns)), "ddp_plan_bucket")
        return ln.value, base.value, fs.value, ns.value

    def slot_param(self, slot: int) -> int:
        p = ctypes.c_int32()
        _check(lib.ddp_plan_slot_param(self._h, slot, ctypes.byref(p)), "ddp_plan_slot_param")
        return p.value

    def param(self, p: int):
        """(bucket, offset within bucket) of parameter p."""
        b, off = ctypes.c_int32(), ctypes.c_int64()
        _check(lib.ddp_plan_param(self._h, p, ctypes.byref(b), ctypes.byref(off)), "ddp_plan_param")
        return b.value, off.value

    def buckets(self) -> List[List[int]]:
        out = []
        for b in range(self.n_buckets):
            _, _, fs, ns = self.bucket(b)
            out.append([self.slot_param(s) for s in range(fs, fs + ns)])
        return out

    def set_occupancy(self, policy):
        """This plan's occupancy policy for the calls that take it:
        "tuned", "shared" or "default" (follow the process-wide one)."""
        _check(lib.ddp_plan_set_occupancy(self._h, _OCCUPANCY[policy]), "ddp_plan_set_occupancy")

    def get_occupancy(self) -> str:
        return _OCCUPANCY_NAME[lib.ddp_plan_get_occupancy(self._h)]

    def prepare(self, n_ranks: Optional[int] = None):
        """Upload the plan's device tables now (``ddp_plan_prepare``), and with
        ``n_ranks`` also the RING table for that rank count
        (``ddp_plan_prepare_ranks``), e.g. before capturing a graph."""
        if n_ranks is None:
            _check(lib.ddp_plan_prepare(self._h), "ddp_plan_prepare")
        else:
            _check(lib.ddp_plan_prepare_ranks(self._h, int(n_ranks)), "ddp_plan_prepare_ranks")


def plan_buckets(numel: Sequence[int], bucket_cap_bytes: int, dtype="f32") -> Plan:
    arr = (ctypes.c_int64 * len(numel))(*numel)
    h = ctypes.c_void_p()
    dt = _DTYPES[dtype]
    _check(lib.ddp_plan_buckets(arr, len(numel), int(bucket_cap_bytes), dt, ctypes.byref(h)),
           "ddp_plan_buckets")
    return Plan(h, dt, numel)


def plan_two_bucket(numel: Sequence[int], region: Sequence[int], dtype="f32") -> Plan:
    arr = (ctypes.c_int64 * len(numel))(*numel)
    reg = (ctypes.c_uint8 * len(region))(*region)
    h = ctypes.c_void_p()
    dt = _DTYPES[dtype]
    _check(lib.ddp_plan_two_bucket(arr, reg, len(numel), dt, ctypes.byref(h)),
           "ddp_plan_two_bucket")
    return Plan(h, dt, numel)


# ---------------------------------------------------------------- bindings

class Binding:
    """Owner of a ``ddp_binding_t`` (one rank's parameter gradient pointers).
    Keeps references to the tensors so their memory outlives the binding."""

    def __init__(self, plan: Plan, grads: Sequence, stream=None):
        self.plan = plan
        self._grads = list(grads)
        if len(self._grads) != len(plan.numel):
            raise ValueError("one gradient tensor per parameter is required")
        for g, n in zip(self._grads, plan.numel):
            if g.numel() != n:
                raise ValueError(f"gradient has {g.numel()} elements, the plan says {n}")
        self.dtypes = {_dtype_code(g) for g in self._grads}
        ptrs = _ptr_array([_dev_ptr(g) for g in self._grads])
        h = ctypes.c_void_p()
        _check(lib.ddp_bind_params(plan.handle, ptrs, ctypes.c_void_p(_stream_handle(stream)),
                                   ctypes.byref(h)), "ddp_bind_params")
        self._h = h

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and lib is not None:
            lib.ddp_binding_free(h)


def bind_params(plan: Plan, grads: Sequence, stream=None) -> Binding:
    return Binding(plan, grads, stream)


class ParamSync:
    """Owner of a ``ddp_param_sync_t``: the synchronisation of one step over
    per-parameter tensors -- every rank's bound gradients averaged straight
    into the per-parameter outputs of ``out_binding``, in one launch, with the
    bits of flatten + sync_allreduce_avg + unflatten.  Keeps the bindings (and
    so their tensors) alive; calling it enqueues the sync."""

    def __init__(self, plan: Plan, rank_bindings: Sequence[Binding], out_binding: Binding,
                 order="ring"):
        self.plan = plan
        self._binds = list(rank_bindings)
        self._out = out_binding
        for bd in self._binds:
            if bd.dtypes != {plan.dtype}:
                raise ValueError("rank gradients must have the plan's dtype")
        if len(out_binding.dtypes) != 1:
            raise ValueError("the outputs must share one dtype")
        self.out_dtype = next(iter(out_binding.dtypes))
        handles = (ctypes.c_void_p * len(self._binds))(*[bd.handle for bd in self._binds])
        h = ctypes.c_void_p()
        _check(lib.ddp_param_sync_create(plan.handle, handles, len(self._binds),
                                         out_binding.handle, _ORDERS[order], self.out_dtype,
                                         ctypes.byref(h)), "ddp_param_sync_create")
        self._h = h

    def __call__(self, stream=None, buckets=None):
        """Enqueues the sync; buckets=(first, count) limits it to those buckets."""
        if buckets is None:
            _check(lib.ddp_param_sync_run(self._h, _stream_handle(stream)), "ddp_param_sync_run")
        else:
            _check(lib.ddp_param_sync_run_buckets(self._h, int(buckets[0]), int(buckets[1]),
                                                  _stream_handle(stream)),
                   "ddp_param_sync_run_buckets")

    def set_occupancy(self, policy):
        """This sync's occupancy policy: "tuned", "shared" or "default"."""
        _check(lib.ddp_param_sync_set_occupancy(self._h, _OCCUPANCY[policy]),
               "ddp_param_sync_set_occupancy")

    def get_occupancy(self) -> str:
        return _OCCUPANCY_NAME[lib.ddp_param_sync_get_occupancy(self._h)]

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and lib is not None:
            lib.ddp_param_sync_free(h)


def param_sync(plan: Plan, rank_bindings: Sequence[Binding], out_binding: Binding,
               order="ring") -> ParamSync:
    return ParamSync(plan, rank_bindings, out_binding, order)


class ParamSGD:
    """Owner of a ``ddp_param_sync_t`` made by ``ddp_param_sgd_create``: every
    rank's bound gradients averaged and folded into an SGD step on the bound
    per-parameter f32 ``params`` (and ``momentum`` buffers), optionally storing
    the average in ``grad_out``.  Calling it with (lr, momentum) enqueues one
    step.  Keeps every binding (and so its tensors) alive."""

    def __init__(self, plan: Plan, rank_bindings: Sequence[Binding], params: Binding,
                 momentum: Optional[Binding] = None, grad_out: Optional[Binding] = None,
                 order="ring", out_dtype=None):
        self.plan = plan
        self._keep = [list(rank_bindings), params, momentum, grad_out]
        for bd in rank_bindings:
            if bd.dtypes != {plan.dtype}:
                raise ValueError("rank gradients must have the plan's dtype")
        for bd in (params, momentum):
            if bd is not None and bd.dtypes != {F32}:
                raise ValueError("parameters and momentum must be float32")
        if grad_out is not None:
            if len(grad_out.dtypes) != 1:
                raise ValueError("the averaged gradients must share one dtype")
            out_dt = next(iter(grad_out.dtypes))
        elif out_dtype is None:
            out_dt = plan.dtype
        elif out_dtype in ("f32", "bf16"):
            out_dt = BF16 if out_dtype == "bf16" else F32
        else:
            raise ValueError(f"unknown out_dtype {out_dtype!r}")
        self.out_dtype = out_dt
        handles = (ctypes.c_void_p * len(rank_bindings))(*[bd.handle for bd in rank_bindings])
        h = ctypes.c_void_p()
        _check(lib.ddp_param_sgd_create(plan.handle, handles, len(rank_bindings),
                                        grad_out.handle if grad_out is not None else None,
                                        params.handle,
                                        momentum.handle if momentum is not None else None,
                                        _ORDERS[order], out_dt, ctypes.byref(h)),
               "ddp_param_sgd_create")
        self._h = h

    def __call__(self, lr: float, momentum: float = 0.0, stream=None, buckets=None):
        """One step; buckets=(first, count) limits it to those buckets."""
        if buckets is None:
            _check(lib.ddp_param_sgd_run(self._h, lr, momentum, _stream_handle(stream)),
                   "ddp_param_sgd_run")
        else:
            _check(lib.ddp_param_sgd_run_buckets(self._h, int(buckets[0]), int(buckets[1]), lr,
                                                 momentum, _stream_handle(stream)),
                   "ddp_param_sgd_run_buckets")

    def set_occupancy(self, policy):
        """This sync's occupancy policy: "tuned", "shared" or "default"."""
        _check(lib.ddp_param_sync_set_occupancy(self._h, _OCCUPANCY[policy]),
               "ddp_param_sync_set_occupancy")

    def get_occupancy(self) -> str:
        return _OCCUPANCY_NAME[lib.ddp_param_sync_get_occupancy(self._h)]

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and lib is not None:
            lib.ddp_param_sync_free(h)


def param_sgd(plan: Plan, rank_bindings: Sequence[Binding], params: Binding,
              momentum: Optional[Binding] = None, grad_out: Optional[Binding] = None,
              order="ring", out_dtype=None) -> ParamSGD:
    return ParamSGD(plan, rank_bindings, params, momentum, grad_out, order, out_dtype)


def _check_flat(plan: Plan, binding: Binding, flat):
    if flat.numel() < plan.total:
        raise ValueError("flat buffer shorter than the plan")
    if binding.dtypes != {_dtype_code(flat)}:
        raise ValueError("flat buffer and parameter gradients differ in dtype")


def flatten(plan: Plan, binding: Binding, flat, bucket: int = -1, stream=None):
    _check_flat(plan, binding, flat)
    _check(lib.ddp_flatten(plan.handle, binding.handle, bucket, _dev_ptr(flat), _dtype_code(flat),
                           _stream_handle(stream)), "ddp_flatten")


def unflatten(plan: Plan, binding: Binding, flat_out, bucket: int = -1, stream=None):
    _check_flat(plan, binding, flat_out)
    _check(lib.ddp_unflatten(plan.handle, binding.handle, bucket, _dev_ptr(flat_out),
                             _dtype_code(flat_out), _stream_handle(stream)), "ddp_unflatten")


# ---------------------------------------------------------------- reduce

def bucket_allreduce_avg(rank_bufs: Sequence, out, order="ring", length: Optional[int] = None,
                         stream=None):
    """Average one bucket over len(rank_bufs) virtual ranks into ``out``."""
    n = out.numel() if length is None else int(length)
    in_dt = _dtype_code(rank_bufs[0])
    for t in rank_bufs:
        if _dtype_code(t) != in_dt or t.numel() < n:
            raise ValueError("rank buffers differ in dtype or are too short")
    if out.numel() < n:
        raise ValueError("output too short")
    ptrs = _ptr_array([_dev_ptr(t) for t in rank_bufs])
    _check(lib.ddp_bucket_allreduce_avg(ptrs, len(rank_bufs), n, _ORDERS[order], in_dt,
                                        _dtype_code(out), _dev_ptr(out), _stream_handle(stream)),
           "ddp_bucket_allreduce_avg")


def sync_allreduce_avg(plan: Plan, rank_flats: Sequence, out_flat, order="ring", stream=None):
    """Average every bucket of ``plan`` in one launch."""
    total = plan.total
    for t in rank_flats:
        if _dtype_code(t) != plan.dtype or t.numel() < total:
            raise ValueError("rank flat buffers differ from the plan's dtype or size")
    if out_flat.numel() < total:
        raise ValueError("output too short")
    ptrs = _ptr_array([_dev_ptr(t) for t in rank_flats])
    _check(lib.ddp_sync_allreduce_avg(plan.handle, ptrs, len(rank_flats), _ORDERS[order],
                                      _dtype_code(out_flat), _dev_ptr(out_flat),
                                      _stream_handle(stream)), "ddp_sync_allreduce_avg")


def sync_allreduce_avg_noalloc(plan: Plan, rank_flats: Sequence, out_flat, order="ring",
                               stream=None):
    """sync_allreduce_avg that allocates no device memory: the plan's tables
    are rebuilt on every call in the library's static device buffer
    (``ddp_sync_allreduce_avg_noalloc``; calls that overlap on one device race
    on it)."""
    total = plan.total
    for t in rank_flats:
        if _dtype_code(t) != plan.dtype or t.numel() < total:
            raise ValueError("rank flat buffers differ from the plan's dtype or size")
    if out_flat.numel() < total:
        raise ValueError("output too short")
    ptrs = _ptr_array([_dev_ptr(t) for t in rank_flats])
    _check(lib.ddp_sync_allreduce_avg_noalloc(plan.handle, ptrs, len(rank_flats), _ORDERS[order],
                                              _dtype_code(out_flat), _dev_ptr(out_flat),
                                              _stream_handle(stream)),
           "ddp_sync_allreduce_avg_noalloc")


def sync_allreduce_avg_bucket(plan: Plan, bucket: int, rank_flats: Sequence, out_flat,
                              order="ring", stream=None):
    """Average bucket ``bucket`` of the plan's flat buffers on its own, with the
    plan's occupancy policy (``ddp_sync_allreduce_avg_bucket``)."""
    total = plan.total
    for t in rank_flats:
        if _dtype_code(t) != plan.dtype or t.numel() < total:
            raise ValueError("rank flat buffers differ from the plan's dtype or size")
    if out_flat.numel() < total:
        raise ValueError("output too short")
    ptrs = _ptr_array([_dev_ptr(t) for t in rank_flats])
    _check(lib.ddp_sync_allreduce_avg_bucket(plan.handle, int(bucket), ptrs, len(rank_flats),
                                             _ORDERS[order], _dtype_code(out_flat),
                                             _dev_ptr(out_flat), _stream_handle(stream)),
           "ddp_sync_allreduce_avg_bucket")


class _PreparedSync:
    """A synchronisation with every argument marshalled once; calling it
    issues the one C call (see make_sync)."""

    def __init__(self, plan: Plan, rank_flats: Sequence, out_flat, order, stream):
        total = plan.total
        for t in rank_flats:
            if _dtype_code(t) != plan.dtype or t.numel() < total:
                raise ValueError("rank flat buffers differ from the plan's dtype or size")
        if out_flat.numel() < total:
            raise ValueError("output too short")
        self._keep = (plan, list(rank_flats), out_flat)   # keeps the memory alive
        self._fn = lib.ddp_sync_allreduce_avg
        self._args = (plan.handle, _ptr_array([_dev_ptr(t) for t in rank_flats]),
                      len(rank_flats), _ORDERS[order], _dtype_code(out_flat),
                      ctypes.c_void_p(_dev_ptr(out_flat)), ctypes.c_void_p(_stream_handle(stream)))

    def __call__(self):
        status = self._fn(*self._args)
        if status != 0:
            _check(status, "ddp_sync_allreduce_avg")


def make_sync(plan: Plan, rank_flats: Sequence, out_flat, order="ring", stream=None):
    """Resolve a synchronisation once -- buffers, order, stream -- and return a
    zero-argument callable that enqueues it (a static graph fixes all of
    these for every step).  The callable keeps its tensors alive; it launches
    on the stream that was current (or given) when it was made."""
    if _ORDERS[order] == RING:
        plan.prepare(len(rank_flats))
    return _PreparedSync(plan, rank_flats, out_flat, order, stream)


def sync_sgd_update(plan: Plan, rank_flats: Sequence, params, lr: float, order="ring",
                    grad_out=None, momentum_buf=None, momentum: float = 0.0,
                    out_dtype=None, stream=None):
    """Average every bucket and apply one SGD step to the flat f32 ``params``
    in the same launch (``ddp_sync_sgd_update``)."""
    import torch
    total = plan.total
    for t in rank_flats:
        if _dtype_code(t) != plan.dtype or t.numel() < total:
            raise ValueError("rank flat buffers differ from the plan's dtype or size")
    for t in (params, momentum_buf):
        if t is not None and (t.dtype != torch.float32 or t.numel() < total):
            raise ValueError("parameters and momentum must be float32 of the plan's size")
    if grad_out is not None:
        if grad_out.numel() < total:
            raise ValueError("grad_out too short")
        out_code = _dtype_code(grad_out)
    else:
        out_code = plan.dtype if out_dtype is None else _DTYPES[out_dtype]
    ptrs = _ptr_array([_dev_ptr(t) for t in rank_flats])
    _check(lib.ddp_sync_sgd_update(plan.handle, ptrs, len(rank_flats), _ORDERS[order], out_code,
                                   None if grad_out is None else _dev_ptr(grad_out),
                                   _dev_ptr(params),
                                   None if momentum_buf is None else _dev_ptr(momentum_buf),
                                   float(lr), float(momentum), _stream_handle(stream)),
           "ddp_sync_sgd_update")


def accumulate(dst: Sequence, src: Sequence, length: Optional[int] = None, stream=None):
    """dst[k] += src[k] for every pair, one launch (``ddp_accumulate``)."""
    if len(dst) != len(src) or not dst:
        raise ValueError("one source per destination is required")
    dt = _dtype_code(dst[0])
    n = dst[0].numel() if length is None else int(length)
    for t in list(dst) + list(src):
        if _dtype_code(t) != dt or t.numel() < n:
            raise ValueError("buffers differ in dtype or are too short")
    _check(lib.ddp_accumulate(_ptr_array([_dev_ptr(t) for t in dst]),
                              _ptr_array([_dev_ptr(t) for t in src]), len(dst), n, dt,
                              _stream_handle(stream)), "ddp_accumulate")


def status_string(status: int) -> str:
    return lib.ddp_status_string(status).decode()


def abi_version() -> int:
    return lib.ddp_abi_version()


OCCUPANCY_TUNED = 0
OCCUPANCY_SHARED = 1
OCCUPANCY_DEFAULT = 2
_OCCUPANCY = {"tuned": OCCUPANCY_TUNED, "shared": OCCUPANCY_SHARED, "default": OCCUPANCY_DEFAULT,
              OCCUPANCY_TUNED: OCCUPANCY_TUNED, OCCUPANCY_SHARED: OCCUPANCY_SHARED,
              OCCUPANCY_DEFAULT: OCCUPANCY_DEFAULT}
_OCCUPANCY_NAME = {OCCUPANCY_TUNED: "tuned", OCCUPANCY_SHARED: "shared",
                   OCCUPANCY_DEFAULT: "default"}


def set_occupancy(policy) -> None:
    """``"tuned"`` (default): the streaming kernels run at their measured best
    number of resident blocks per CU; ``"shared"``: no cap, for syncs that
    overlap compute on other streams (``ddp_set_occupancy``).  Process-wide:
    the policy of calls without an object and of objects left at "default"
    (see Plan.set_occupancy, ParamSync.set_occupancy)."""
    if policy not in ("tuned", "shared", OCCUPANCY_TUNED, OCCUPANCY_SHARED):
        raise ValueError(f"unknown occupancy policy {policy!r}")
    _check(lib.ddp_set_occupancy(_OCCUPANCY[policy]), "ddp_set_occupancy")


def get_occupancy() -> str:
    return "tuned" if lib.ddp_get_occupancy() == OCCUPANCY_TUNED else "shared"
