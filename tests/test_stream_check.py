"""Host-side test of the streaming comparator the full-size GPU parity tests
use (tests/gpu_stream.py), on CPU tensors: every element of every run is
handed to the check exactly once, at its own offset, across piece and
sub-range edges; a planted mismatch is reported; the oracle's piece form
checks a bucket streamed this way."""
import threading

import numpy as np
import pytest

import oracle
from gpu_stream import StreamedCheck

torch = pytest.importorskip("torch")


def test_every_element_once_at_its_offset():
    seen = {}
    lock = threading.Lock()

    def check(meta, off, hosts):
        a, b = hosts["a"], hosts["b"]
        assert np.array_equal(a, np.arange(off, off + a.size, dtype=np.float32) + meta)
        assert np.array_equal(b.view(np.uint16), (np.arange(off, off + a.size) % 65536)
                              .astype(np.uint16))
        with lock:
            for i in range(off, off + a.size):
                key = (meta, i)
                assert key not in seen
                seen[key] = True

    runs = {0: 1, 1000: 5000, 2000: 37, 3000: 4096 * 3 + 17}
    with StreamedCheck(torch, check, piece=4096, threads=3, min_sub=1000) as sc:
        for meta, n in runs.items():
            a = torch.arange(n, dtype=torch.float32) + meta
            b = (torch.arange(n) % 65536).to(torch.int32).to(torch.int16).view(torch.bfloat16)
            sc.add(meta, {"a": a, "b": b})
        total = sc.finish()
    assert total == sum(runs.values())
    assert len(seen) == total


def _bucket_check(N, L):
    def check(meta, off, hosts):
        want = oracle.bucket_range_avg([hosts[f"x{r}"] for r in range(N)], L, meta + off, "ring")
        assert np.array_equal(hosts["y"].view(np.uint32), want.view(np.uint32)), (meta, off)
    return check


def test_streamed_bucket_matches_and_a_planted_mismatch_is_found():
    rng = np.random.default_rng(3)
    N, L = 5, 30011
    xs = [rng.standard_normal(L).astype(np.float32) for _ in range(N)]
    y = oracle.bucket_avg(xs, "ring")
    views = {f"x{r}": torch.from_numpy(x) for r, x in enumerate(xs)}
    with StreamedCheck(torch, _bucket_check(N, L), piece=4096, threads=4, min_sub=700) as sc:
        # the bucket handed over as two runs, the second starting inside a chunk
        cut = 7001
        sc.add(0, {**{k: v[:cut] for k, v in views.items()}, "y": torch.from_numpy(y[:cut])})
        sc.add(cut, {**{k: v[cut:] for k, v in views.items()}, "y": torch.from_numpy(y[cut:])})
        assert sc.finish() == L
    bad = y.copy()
    bad[L - 3] = np.nextafter(bad[L - 3], np.float32(1))
    with pytest.raises(AssertionError):
        with StreamedCheck(torch, _bucket_check(N, L), piece=4096, threads=4, min_sub=700) as sc:
            sc.add(0, {**views, "y": torch.from_numpy(bad)})
            sc.finish()
