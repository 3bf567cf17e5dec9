"""The oracle's pins are sharp: each plausible mistake planted in a copy of
the oracle (on the CPU, in a temporary build) makes at least one pin fail,
while the real oracle passes them all.

Mistakes planted in the C core: ring start rank off by one, ring walked
backwards, floor instead of ceil chunking, a rank dropped from the sum, the
scale by 1/(N-1), a -0 start for the sequential sum, round-half-up instead of
ties-to-even, the NaN quiet bit lost, a wrong bf16 widening, the N == 1
identity replaced by the fold, a bucket piece folded as if it began
the bucket.  In the Python layer: forward instead of
reverse packing, closing a bucket when it is exactly full, FIRST_COMM regions
in the wrong order, the simulator forgetting to accumulate, the all-gather
forwarding the wrong chunk.
"""
import os
import re
import subprocess
import sys
import types
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_DIR = os.path.dirname(oracle.__file__)
C_SRC = open(os.path.join(ORACLE_DIR, "oracle_core.c")).read()
PY_SRC = open(os.path.join(ORACLE_DIR, "__init__.py")).read()


# ------------------------------------------------------------------ battery

def _golden():
    tables, cur = {}, None
    for line in open(os.path.join(HERE, "golden", "ring_4gpu_walkthrough.txt"), encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        m = re.match(r"\[(RS|AG) (\d)\]", line)
        if m:
            cur = (m.group(1), int(m.group(2)))
            tables[cur] = []
            continue
        tables[cur].append([c.strip() for c in line.split(":", 1)[1].split("|")])
    return tables


def _cell(cell):
    if cell == ".":
        return None
    if cell.startswith("S"):
        return float(sum(2 ** (4 * i + int(cell[1:])) for i in range(4)))
    return float(sum(2 ** (4 * int(t[0]) + int(t[1])) for t in cell.split("+")))


def pin_p1_tables(o):
    A = [np.array([2.0 ** (4 * i + j) for j in range(4)], np.float32) for i in range(4)]
    res = o.ring_allreduce(A, s0=0, trace=True)
    tab = _golden()
    for ph, snaps in (("RS", res["rs"]), ("AG", res["ag"])):
        for rnd in (1, 2, 3):
            for g in range(4):
                for c in range(4):
                    want = _cell(tab[(ph, rnd)][g][c])
                    if want is not None and float(snaps[rnd - 1][g][c]) != want:
                        return False
    return True


def pin_p2_zero_start(o):
    z = np.array([-0.0] * 5, np.float32)
    return not np.signbit(o.bucket_avg([z, z, z], "seq")).any() and \
        np.signbit(o.bucket_avg([z, z, z], "ring")).all()


def pin_p3_identity(o):
    rng = np.random.default_rng(0)
    for N in (2, 4, 8):
        B, L = 4 * N, 9
        d = [[Fraction(int(v), 256) for v in rng.integers(-64, 65, L)] for _ in range(B)]
        m = B // N
        xs = [np.array([float(Fraction(N, B) * sum(d[i][j] for i in range(k * m, (k + 1) * m)))
                        for j in range(L)], np.float32) for k in range(N)]
        full = [sum(d[i][j] for i in range(B)) / B for j in range(L)]
        for order in ("seq", "ring"):
            got = o.bucket_avg(xs, order)
            if any(Fraction(float(g)) != f for g, f in zip(got, full)):
                return False
    return True


def pin_p5_simulator(o):
    rng = np.random.default_rng(1)
    for N in (3, 4, 5):
        for L in (7, 13, 20):
            bufs = [rng.standard_normal(L).astype(np.float32) for _ in range(N)]
            sim = o.ring_allreduce_avg(bufs, s0=1)
            closed = o.bucket_avg(bufs, "ring")
            if any(not np.array_equal(s.view(np.uint32), closed.view(np.uint32)) for s in sim):
                return False
    return True


def pin_p8_rne(o):
    hi = (np.arange(0, 1 << 16, 7, dtype=np.uint32) << np.uint32(16))
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    fin = (u & np.uint32(0x7F800000)) != np.uint32(0x7F800000)
    x = u[fin].view(np.float32)
    torch = pytest.importorskip("torch")
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if not np.array_equal(o.rne_bf16(x), want):
        return False
    nan = np.array([0x7F800001, 0xFF800001, 0x7FC00000], np.uint32).view(np.float32)
    g = o.rne_bf16(nan)
    return bool((((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)).all())


def pin_p9_scale(o):
    x = np.random.default_rng(2).standard_normal(500).astype(np.float32)
    for N in (2, 4, 8):
        xs = [x] + [np.zeros_like(x)] * (N - 1)
        if not np.array_equal(o.bucket_avg(xs, "ring").view(np.uint32),
                              (x / np.float32(N)).astype(np.float32).view(np.uint32)):
            return False
    return True


def pin_p10_single(o):
    pats = np.array([0x80000000, 0x7FC00123, 0x00000001, 0x3F800000], np.uint32)
    return all(np.array_equal(o.bucket_avg([pats.view(np.float32)], order).view(np.uint32), pats)
               for order in ("seq", "ring"))


def pin_bf16_path(o):
    rng = np.random.default_rng(3)
    hs = [(rng.integers(0, 1 << 16, 300, dtype=np.uint32) & 0xBFFF).astype(np.uint16)
          for _ in range(4)]
    wid = [(h.astype(np.uint32) << np.uint32(16)).view(np.float32) for h in hs]
    return np.array_equal(o.bucket_avg(hs, "ring", "bf16", "bf16"),
                          o.rne_bf16(o.bucket_avg(wid, "ring", "f32", "f32")))


def pin_p7_plans(o):
    ok = o.plan_cap([3, 5, 2, 7, 1], 40, 4).buckets == [[4, 3, 2], [1, 0]]
    ok &= o.plan_cap([5, 5, 5], 40, 4).buckets == [[2, 1], [0]]
    ok &= o.plan_cap([100, 1, 1], 40, 4).buckets == [[2, 1], [0]]
    regs = [o.FIRST, o.BN_WEIGHT, o.BN_BIAS, o.DEEP, o.FC_WEIGHT, o.FC_BIAS, o.DEEP]
    ok &= o.plan_two_bucket([1] * 7, regs).buckets == [[3, 6], [2, 1, 5, 4, 0]]
    return ok


def pin_sgd(o):
    p = np.array([1.0, -2.0, 0.5], np.float32)
    m = np.zeros(3, np.float32)
    o.sgd_step(p, np.array([0.5, 0.25, -1.0], np.float32), 0.5, momentum_buf=m, momentum=0.5)
    o.sgd_step(p, np.array([1.0, 1.0, 1.0], np.float32), 0.5, momentum_buf=m, momentum=0.5)
    # v1 = g1; p1 = p0 - v1/2; v2 = v1/2 + g2; p2 = p1 - v2/2
    return p.tolist() == [0.125, -2.6875, 0.75] and m.tolist() == [1.25, 1.125, 0.5]


def pin_sampled(o):
    rng = np.random.default_rng(4)
    x = [rng.standard_normal(50).astype(np.float32) for _ in range(3)]
    whole = o.bucket_avg(x, "ring")
    pos = np.array([0, 16, 17, 33, 34, 49])
    vals = np.stack([np.array([x[r][i] for r in range(3)]) for i in pos])
    got = o.sampled_avg(vals, pos, np.full(pos.size, 50), "ring")
    return np.array_equal(got.view(np.uint32), whole[pos].view(np.uint32))


def pin_bucket_pieces(o):
    rng = np.random.default_rng(5)
    x = [rng.standard_normal(50).astype(np.float32) for _ in range(3)]
    whole = o.bucket_avg(x, "ring")
    got = np.concatenate([o.bucket_range_avg([v[a:b] for v in x], 50, a, "ring")
                          for a, b in ((0, 10), (10, 30), (30, 50))])
    return np.array_equal(got.view(np.uint32), whole.view(np.uint32))


def pin_flatten(o):
    sizes = [3, 5, 2, 4]
    plan = o.plan_cap(sizes, 24, 4)
    grads = [np.array([10 * p + j for j in range(n)], np.float32) for p, n in enumerate(sizes)]
    return o.flatten(plan, grads).tolist() == [30, 31, 32, 33, 20, 21, 10, 11, 12, 13, 14, 0, 1, 2]


def pin_accumulate(o):
    d = np.array([1.0, 2.5, -3.0], np.float32)
    o.accumulate(d, np.array([0.5, 0.5, 1.0], np.float32))
    return d.tolist() == [1.5, 3.0, -2.0]


BATTERY = [pin_sampled, pin_bucket_pieces, pin_flatten, pin_accumulate, pin_sgd, pin_p1_tables, pin_p2_zero_start, pin_p3_identity, pin_p5_simulator, pin_p8_rne,
           pin_p9_scale, pin_p10_single, pin_bf16_path, pin_p7_plans]


def run_battery(o):
    failed = []
    for pin in BATTERY:
        try:
            ok = pin(o)
        except Exception:           # a mutant may also raise: that is a failed pin
            ok = False
        if not ok:
            failed.append(pin.__name__)
    return failed


# ------------------------------------------------------------------ mutants

C_MUTANTS = {
    "ring_start_off_by_one": ("return (int)((c + 1) % N);", "return (int)(c % N);"),
    "ring_walked_backwards": ("acc = acc + v[(s + k) % N];", "acc = acc + v[(s - k + N) % N];"),
    "floor_chunks": ("int64_t C = (len + N - 1) / N;", "int64_t C = (len + N) / N;"),
    "rank_dropped": ("for (int r = 0; r < N; ++r) acc = acc + v[r];",
                     "for (int r = 0; r < N - 1; ++r) acc = acc + v[r];"),
    "scale_by_n_minus_1": ("const float inv = 1.0f / (float)N;\n    float v[1024];\n    for (int64_t i",
                           "const float inv = 1.0f / (float)(N - 1);\n    float v[1024];\n    for (int64_t i"),
    "negative_zero_start": ("acc = 0.0f;", "acc = -0.0f;"),
    "round_half_up": ("if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))",
                      "if (lower >= 0x8000u)"),
    "nan_quiet_bit_lost": ("return (uint16_t)((u >> 16) | 0x0040u);", "return (uint16_t)(u >> 16);"),
    "bad_bf16_widen": ("return bits_to_f32((uint32_t)h << 16);", "return bits_to_f32((uint32_t)h << 15);"),
    "single_rank_folds": ("    if (N == 1) {\n        if (in_dtype != out_dtype) return -1;\n        memcpy",
                          "    if (N == -1) {\n        if (in_dtype != out_dtype) return -1;\n        memcpy"),
    "accumulate_subtracts": ("store_elem(dst, dtype, i, a + b);", "store_elem(dst, dtype, i, a - b);"),
    "sgd_sign_flipped": ("p[i] = p[i] - step;", "p[i] = p[i] + step;"),
    "sampled_rows_rank_major": ("v[r] = load_elem(vals, in_dtype, s * N + r);",
                                "v[r] = load_elem(vals, in_dtype, r * S + s);"),
    "piece_positions_from_zero": ("float acc = fold(v, N, order, lo + k, len);",
                                  "float acc = fold(v, N, order, k, len);"),
    "sgd_momentum_terms_swapped": ("float v = mu * m[i];\n            v = v + gi;",
                                   "float v = mu * gi;\n            v = v + m[i];"),
}

PY_MUTANTS = {
    "forward_packing": ("for p in reversed(range(len(numel))):", "for p in range(len(numel)):"),
    "close_when_full": ("if cur and cur_bytes + nb > bucket_cap_bytes:",
                        "if cur and cur_bytes + nb >= bucket_cap_bytes:"),
    "first_comm_region_order": ("first = [p for reg in FIRST_COMM_REGIONS for p",
                                "first = [p for reg in FIRST_COMM_REGIONS[::-1] for p"),
    "simulator_no_accumulate": ("b[dst][lo:hi] = data + b[dst][lo:hi]", "b[dst][lo:hi] = data"),
    "allgather_wrong_chunk": ("c = (i + 1 - s0 - t) % N", "c = (i - s0 - t) % N"),
    "flatten_in_registration_order": (
        "flat = np.empty(plan.total, dtype=grads[0].dtype)\n"
        "    for b, base in zip(plan.buckets, plan.bucket_base):\n        off = base\n        for p in b:",
        "flat = np.empty(plan.total, dtype=grads[0].dtype)\n"
        "    for b, base in zip(plan.buckets, plan.bucket_base):\n        off = base\n        for p in sorted(b):"),
}


def _c_mutant(tmp_path, name, old, new):
    assert C_SRC.count(old) == 1, name
    src = tmp_path / f"{name}.c"
    lib = tmp_path / f"lib{name}.so"
    src.write_text(C_SRC.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", str(lib), str(src)])
    mod = _module(f"oracle_c_{name}", PY_SRC)
    mod._lib = mod.load_core(str(lib))
    return mod


def _module(name, source):
    """Execute oracle source text as a fresh module (registered so that
    dataclasses can resolve it)."""
    mod = types.ModuleType(name)
    mod.__dict__["__file__"] = oracle.__file__
    sys.modules[name] = mod
    exec(compile(source, oracle.__file__, "exec"), mod.__dict__)
    return mod


def _py_mutant(name, old, new):
    assert PY_SRC.count(old) == 1, name
    return _module(f"oracle_py_{name}", PY_SRC.replace(old, new))


def test_real_oracle_passes_the_battery():
    assert run_battery(oracle) == []


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_core_mutant_is_caught(tmp_path, name):
    mod = _c_mutant(tmp_path, name, *C_MUTANTS[name])
    assert run_battery(mod), f"no pin caught {name}"


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_mutant_is_caught(name):
    mod = _py_mutant(name, *PY_MUTANTS[name])
    assert run_battery(mod), f"no pin caught {name}"
