"""Helpers shared by the GPU parity tests (host <-> device marshalling and
bitwise comparison; no arithmetic of the method)."""
import numpy as np
import pytest


def torch_cuda():
    torch = pytest.importorskip("torch")
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch


def to_dev(a, torch, device="cuda:0"):
    """numpy float32 -> float32 tensor; numpy uint16 (bf16 patterns) -> bfloat16 tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32, copy=False).copy()).to(device)


def to_host(t, torch):
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def _nan_mask(a):
    if a.dtype == np.uint16:
        return ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
    return np.isnan(a)


def assert_bits_equal(got, want, what=""):
    """Bitwise equality; NaNs compared by class (payloads are not fixed by IEEE-754)."""
    assert got.dtype == want.dtype and got.shape == want.shape, (got.dtype, want.dtype, got.shape,
                                                                  want.shape)
    gn, wn = _nan_mask(got), _nan_mask(want)
    bad_nan = np.nonzero(gn != wn)[0]
    assert bad_nan.size == 0, f"{what}: NaN class differs at {bad_nan[:8]}"
    view = np.uint16 if got.dtype == np.uint16 else np.uint32
    gb, wb = got.view(view), want.view(view)
    bad = np.nonzero((gb != wb) & ~gn)[0]
    assert bad.size == 0, (f"{what}: {bad.size} elements differ, first at {bad[:8]}: "
                           f"got {[hex(int(x)) for x in gb[bad[:4]]]} "
                           f"want {[hex(int(x)) for x in wb[bad[:4]]]}")


def random_inputs(rng, n_ranks, length, dtype, scale=1e-3):
    """Seeded rank buffers: float32 normals, or finite bf16 bit patterns."""
    if dtype == "f32":
        return [(rng.standard_normal(length) * scale).astype(np.float32) for _ in range(n_ranks)]
    out = []
    for _ in range(n_ranks):
        f = (rng.standard_normal(length) * scale).astype(np.float32)
        out.append((f.view(np.uint32) >> np.uint32(16)).astype(np.uint16))
    return out


def sample_positions(bucket_base, bucket_len, n_ranks, total, rng, n_random=20000):
    """Element positions that cover every bucket edge and ring chunk edge,
    plus uniform random positions."""
    pos = set()
    for base, ln in zip(bucket_base, bucket_len):
        if ln == 0:
            continue
        C = -(-ln // n_ranks)
        for k in range(n_ranks + 1):
            e = base + min(k * C, ln)
            for d in (-9, -5, -2, -1, 0, 1, 2, 5, 8):
                if base <= e + d < base + ln:
                    pos.add(e + d)
    pos.update(int(x) for x in rng.integers(0, total, n_random))
    return np.array(sorted(pos), dtype=np.int64)
