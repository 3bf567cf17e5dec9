"""Full-size comparison of device results with the oracle, piece by piece.

Multi-GB workloads do not fit the host as whole rank sets, so every output
element is checked by streaming: each piece of a run of elements is copied
device -> pinned host memory (every named tensor of the piece), and host
threads run the caller's check on sub-ranges of it (the oracle's C calls
release the GIL) while the next piece is copied.  No arithmetic of the
method lives here: the check function calls the oracle.
"""
import contextlib
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

PIECE = 1 << 24          # elements per copied piece
MIN_SUB = 1 << 19        # smallest sub-range handed to one host thread


def host_threads():
    """Host threads to use: the CPUs this process may run on, at most 16
    (a host shared by several GPUs gives each a share of its CPUs)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _np_view(t, torch):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class StreamedCheck:
    """Streams runs of elements to the host and checks them on threads.

    ``add(meta, views)``: ``views`` maps names to 1-D device tensors of one
    length (slices of rank buffers, outputs, parameters...).  For every piece
    [a, a + n) of them and every sub-range of that piece, the check function
    is called as ``check(meta, off, hosts)`` with ``off`` the sub-range's
    offset in the run and ``hosts`` mapping each name to the host copy of the
    sub-range (numpy; bf16 as uint16 bit patterns).  It raises on a mismatch.
    ``finish()`` waits for every check and re-raises the first failure.
    Device work producing the views must be complete (synchronised) before
    ``add`` is called."""

    def __init__(self, torch, check, piece=PIECE, slots=3, threads=None, min_sub=MIN_SUB):
        self.torch, self.check, self.piece, self.min_sub = torch, check, piece, min_sub
        self.threads = threads or host_threads()
        self.pool = ThreadPoolExecutor(self.threads)
        self.slots = [dict() for _ in range(slots)]
        self.pending = [[] for _ in range(slots)]
        self.next_slot = 0
        # CPU tensors (the host-side test of this helper) take plain copies
        self.on_gpu = torch.cuda.is_available()
        self.copy_stream = torch.cuda.Stream() if self.on_gpu else None
        self.elements = 0
        self.failure = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        if self.slots is not None:
            self.pool.shutdown(wait=True, cancel_futures=True)
            self.slots = None
        return False

    def _buffer(self, slot, name, dtype):
        buf = self.slots[slot].get(name)
        if buf is None or buf.dtype != dtype:
            buf = self.torch.empty(self.piece, dtype=dtype, pin_memory=self.on_gpu)
            self.slots[slot][name] = buf
        return buf

    def _drain(self, slot):
        for f in self.pending[slot]:
            exc = f.exception()
            if exc is not None and self.failure is None:
                self.failure = exc
        self.pending[slot] = []
        if self.failure is not None:
            raise self.failure

    def add(self, meta, views):
        torch = self.torch
        n_all = {v.numel() for v in views.values()}
        assert len(n_all) == 1, f"views differ in length: {n_all}"
        n_all = n_all.pop()
        for a in range(0, n_all, self.piece):
            n = min(self.piece, n_all - a)
            slot = self.next_slot
            self.next_slot = (slot + 1) % len(self.slots)
            self._drain(slot)
            hosts = {}
            ctx = torch.cuda.stream(self.copy_stream) if self.on_gpu else contextlib.nullcontext()
            with ctx:
                for name, v in views.items():
                    buf = self._buffer(slot, name, v.dtype)
                    buf[:n].copy_(v[a:a + n], non_blocking=self.on_gpu)
                    hosts[name] = _np_view(buf, torch)
            if self.on_gpu:
                self.copy_stream.synchronize()
            sub = max(self.min_sub, -(-n // self.threads))
            for s in range(0, n, sub):
                e = min(n, s + sub)
                part = {k: h[s:e] for k, h in hosts.items()}
                self.pending[slot].append(self.pool.submit(self.check, meta, a + s, part))
            self.elements += n

    def finish(self):
        try:
            for slot in range(len(self.slots)):
                self._drain(slot)
        finally:
            self.pool.shutdown(wait=True)
            self.slots = None
        return self.elements
