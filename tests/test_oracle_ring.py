"""Pins of the oracle's ring order against the page "DDP" (sgdbs.github.io,
AI_Infra/1.DataParallel), sections 2.8-2.12.

* P1  the literal simulator reproduces the printed 4-GPU tables round by round
      (start offset 0, the tables' convention), and the relabelled version
      (start offset 1) makes rank c own sigma_c.
* P5  AllReduce = ReduceScatter + AllGather: after the all-gather every rank
      holds the same buffer, equal bit for bit to the oracle's closed-form
      ring fold (start offset 1).
* P6  2(N-1) rounds and 2(N-1)/N * L elements sent per rank.
* P4  with exact (small integer) inputs the ring and sequential orders agree.
"""
import os
import re

import numpy as np
import pytest

import oracle


def _parse_golden(path):
    tables, cur = {}, None
    for line in open(path, encoding="utf-8"):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        m = re.match(r"\[(RS|AG) (\d)\]", line)
        if m:
            cur = (m.group(1), int(m.group(2)))
            tables[cur] = []
            continue
        gpu, cells = line.split(":", 1)
        tables[cur].append([c.strip() for c in cells.split("|")])
    return tables


def _value_of(cell):
    """Exact value of a cell with A_ij = 2**(4i+j); None for '.'."""
    if cell == ".":
        return None
    if cell.startswith("S"):
        j = int(cell[1:])
        return float(sum(2 ** (4 * i + j) for i in range(4)))
    return float(sum(2 ** (4 * int(t[0]) + int(t[1])) for t in cell.split("+")))


def _A():
    # GPU i, chunk j (chunk length 1): A_ij = 2**(4i+j); 16 distinct powers of
    # two, so every partial sum is exact and names the terms it contains.
    return [np.array([2.0 ** (4 * i + j) for j in range(4)], dtype=np.float32) for i in range(4)]


def test_p1_printed_tables_round_by_round(golden_dir):
    tables = _parse_golden(os.path.join(golden_dir, "ring_4gpu_walkthrough.txt"))
    res = oracle.ring_allreduce(_A(), s0=0, trace=True)
    sigma = [float(sum(2 ** (4 * i + j) for i in range(4))) for j in range(4)]
    for phase, snaps in (("RS", res["rs"]), ("AG", res["ag"])):
        for rnd in (1, 2, 3):
            table = tables[(phase, rnd)]
            for gpu in range(4):
                for chunk in range(4):
                    got = float(snaps[rnd - 1][gpu][chunk])
                    want = _value_of(table[gpu][chunk])
                    if want is None:
                        assert got != sigma[chunk], (phase, rnd, gpu, chunk)
                    else:
                        assert got == want, (phase, rnd, gpu, chunk, got, want)
    # owners after Phase 1 as the text states them
    assert res["owner_chunk"] == [1, 2, 3, 0]
    assert res["rounds"] == 6


def test_p1_relabelled_start_offset_one_owner_is_chunk_index():
    res = oracle.ring_allreduce(_A(), s0=1, trace=True)
    rs_last = res["rs"][-1]
    for c in range(4):
        assert float(rs_last[c][c]) == float(sum(2 ** (4 * i + c) for i in range(4)))
    assert res["owner_chunk"] == [0, 1, 2, 3]


@pytest.mark.parametrize("N", [2, 3, 4, 5, 7, 8])
@pytest.mark.parametrize("L", [0, 1, 2, 5, 13, 64, 1001])
def test_p5_allgather_of_reducescatter_equals_closed_form(N, L):
    rng = np.random.default_rng(1000 * N + L)
    bufs = [rng.standard_normal(L).astype(np.float32) * np.float32(1e-3) for _ in range(N)]
    res = oracle.ring_allreduce(bufs, s0=1)
    final = res["final"]
    for r in range(1, N):
        assert np.array_equal(final[r].view(np.uint32), final[0].view(np.uint32))
    avg = oracle.ring_allreduce_avg(bufs, s0=1)
    closed = oracle.bucket_avg(bufs, oracle.RING)
    for r in range(N):
        assert np.array_equal(avg[r].view(np.uint32), closed.view(np.uint32))


@pytest.mark.parametrize("N", [2, 3, 4, 8])
def test_p5_owner_chunk_after_reduce_scatter_is_the_full_sum(N):
    L = 10 * N + 3
    rng = np.random.default_rng(N)
    bufs = [rng.standard_normal(L).astype(np.float32) for _ in range(N)]
    res = oracle.ring_allreduce(bufs, s0=1, trace=True)
    after_rs = res["rs"][-1]
    for i in range(N):
        c = res["owner_chunk"][i]
        lo, hi = res["chunks"][c]
        # the owner's chunk is final after reduce-scatter: all-gather only copies it
        assert np.array_equal(after_rs[i][lo:hi].view(np.uint32),
                              res["final"][0][lo:hi].view(np.uint32))


@pytest.mark.parametrize("N", [2, 3, 4, 6, 8])
def test_p6_rounds_and_traffic(N):
    L = 12 * N
    bufs = [np.ones(L, dtype=np.float32)] * N
    res = oracle.ring_allreduce(bufs, s0=1)
    assert res["rounds"] == 2 * (N - 1)
    # traffic_per_rank = 2 (N-1)/N |g|  ("(24) NCCL通信与分布式数据并行", section 十四;
    # "DDP" section 2.12)
    for s in res["sent"]:
        assert s == 2 * (N - 1) * L // N
        assert s == pytest.approx(2.0 * (N - 1) / N * L)


@pytest.mark.parametrize("N", [2, 3, 5, 8])
def test_p4_exact_inputs_make_orders_agree(N):
    rng = np.random.default_rng(7 + N)
    L = 257
    bufs = [rng.integers(-1000, 1000, L).astype(np.float32) for _ in range(N)]
    seq = oracle.bucket_avg(bufs, oracle.SEQ)
    ring = oracle.bucket_avg(bufs, oracle.RING)
    assert np.array_equal(seq.view(np.uint32), ring.view(np.uint32))


def test_p4_two_ranks_orders_agree_except_signed_zero():
    rng = np.random.default_rng(3)
    a = rng.standard_normal(4097).astype(np.float32)
    b = rng.standard_normal(4097).astype(np.float32)
    seq = oracle.bucket_avg([a, b], oracle.SEQ)
    ring = oracle.bucket_avg([a, b], oracle.RING)
    assert np.array_equal(seq.view(np.uint32), ring.view(np.uint32))
    z = np.array([-0.0], dtype=np.float32)
    assert np.signbit(oracle.bucket_avg([z, z], oracle.RING))[0]
    assert not np.signbit(oracle.bucket_avg([z, z], oracle.SEQ))[0]


def test_ring_order_differs_from_sequential_for_three_or_more_ranks():
    # the two fixed orders are distinct definitions: for N >= 3 they give
    # different bits on some inputs (the pages note that accumulation order
    # changes the last bits, "DDP" section 3.1)
    rng = np.random.default_rng(11)
    bufs = [rng.standard_normal(10000).astype(np.float32) for _ in range(4)]
    seq = oracle.bucket_avg(bufs, oracle.SEQ)
    ring = oracle.bucket_avg(bufs, oracle.RING)
    assert not np.array_equal(seq, ring)
