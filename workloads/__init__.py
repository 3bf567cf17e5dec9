"""Seeded synthetic workloads for bucketed gradient synchronisation.

This module holds only what both sides of a parity check need to agree on
*before* any arithmetic of the method runs: the parameter shape lists of the
model families the workloads are named after, and seeded random gradient
values.  It computes no bucket plan, no reduction, no scaling and no
rounding of the method; it is imported by the tests, by ``bench.py`` and by
``__graft_entry__.smoke()``, never by ``oracle/`` or by the HIP library.

Generators
----------
* ``philox4x32_10`` — the counter-based generator of Salmon, Moraes, Dror and
  Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11), 10 rounds,
  written from its published definition (multipliers 0xD2511F53 /
  0xCD9E8D57, Weyl key bumps 0x9E3779B9 / 0xBB67AE85).
* ``normal_f32`` — Box-Muller in double precision on two 53-bit uniforms taken
  from one Philox block, scaled by sigma (the standard deviation) and rounded
  once to float32.  Element ``i`` of a stream is component ``i % 2`` of block
  ``i // 2`` with counter ``(i//2 low, i//2 high, stream, 0)`` and key
  ``(seed low, seed high)``.
* ``device_normal_`` — for the full-size workloads (tens of GB of gradients)
  the values are drawn on the GPU by torch's own seeded generator; these
  never feed a stored expected value, only sampled GPU/oracle comparisons in
  which the oracle reads the same device values back.

Seeds follow the per-rank seeding idiom of the page "DDP"
(sgdbs.github.io, AI_Infra/1.DataParallel, section 4.3 on per-rank
seeds): virtual rank ``r`` uses ``base_seed + r``.

Shapes
------
Registration (forward) order, as ``module.parameters()`` would list them.
Region tags name the gradient regions of the two-bucket split of
"(24) NCCL通信与分布式数据并行" (tech-renaissance.cn), section 七 (G-series
regions) and section 八 (DEEP_COMM / FIRST_COMM).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# Region tags for the two-bucket split (values are the ABI's numbering).
# ---------------------------------------------------------------------------
REGION_BN_BIAS = 0
REGION_BN_WEIGHT = 1
REGION_FC_BIAS = 2
REGION_FC_WEIGHT = 3
REGION_FIRST = 4
REGION_DEEP = 5

MiB = 1 << 20


@dataclass(frozen=True)
class Param:
    name: str
    numel: int
    region: int


# ---------------------------------------------------------------------------
# Philox4x32-10 (Salmon et al., SC'11)
# ---------------------------------------------------------------------------
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Ten Philox rounds on uint32 counters held in uint64 arrays.

    Returns the four output words as uint64 arrays with values < 2**32.
    """
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    ka, kb = k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            ka = (ka + _W0) & 0xFFFFFFFF
            kb = (kb + _W1) & 0xFFFFFFFF
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> _S32, p0 & _MASK
        hi1, lo1 = p1 >> _S32, p1 & _MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(ka), lo1,
                          hi0 ^ c3 ^ np.uint64(kb), lo0)
    return c0, c1, c2, c3


def _blocks(seed: int, stream: int, first_block: int, n_blocks: int):
    j = np.arange(first_block, first_block + n_blocks, dtype=np.uint64)
    zeros = np.zeros_like(j)
    return philox4x32_10(j & _MASK, j >> _S32, zeros + np.uint64(stream & 0xFFFFFFFF),
                         zeros, seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)


def _unit_open(lo, hi):
    """53-bit uniform in (0, 1) from two 32-bit words."""
    bits = ((hi << _S32) | lo) >> np.uint64(11)
    return (bits.astype(np.float64) + 0.5) * (2.0 ** -53)


def uniform_f64(seed: int, stream: int, n: int) -> np.ndarray:
    """n uniforms in (0,1); element i uses words 0,1 of block i."""
    w0, w1, _, _ = _blocks(seed, stream, 0, n)
    return _unit_open(w0, w1)


def normal_f32(seed: int, stream: int, n: int, sigma: float,
               offset: int = 0) -> np.ndarray:
    """n Normal(0, sigma) float32 values, elements [offset, offset+n) of a stream."""
    if n <= 0:
        return np.zeros(0, dtype=np.float32)
    b0 = offset // 2
    b1 = (offset + n + 1) // 2
    w0, w1, w2, w3 = _blocks(seed, stream, b0, b1 - b0)
    u1 = _unit_open(w0, w1)
    u2 = _unit_open(w2, w3)
    r = np.sqrt(-2.0 * np.log(u1))
    th = 2.0 * math.pi * u2
    z = np.empty(2 * (b1 - b0), dtype=np.float64)
    z[0::2] = r * np.cos(th)
    z[1::2] = r * np.sin(th)
    start = offset - 2 * b0
    return (z[start:start + n] * sigma).astype(np.float32)


def f32_to_bf16_bits_input(x: np.ndarray) -> np.ndarray:
    """Input preparation for the bf16 workloads: draw in float32, keep the
    nearest bf16 (ties to even) as the stored gradient.  This only makes the
    *input* values; no result of the method passes through here.  NaN inputs
    are not produced by the generators."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


# ---------------------------------------------------------------------------
# Shape lists (registration order)
# ---------------------------------------------------------------------------

def tiny_linear() -> List[Param]:
    """nn.Linear(128, 10): weight 10x128 registered before bias 10."""
    return [Param("weight", 10 * 128, REGION_FC_WEIGHT),
            Param("bias", 10, REGION_FC_BIAS)]


def resnet50() -> List[Param]:
    """Standard ResNet-50 parameter list: stem, 16 bottlenecks in stages
    [3, 4, 6, 3] with mid widths 64/128/256/512 and expansion 4 (first block
    of each stage adds a 1x1 downsample conv + BN), then fc 1000x2048 + bias.
    161 tensors, 25,557,032 elements."""
    ps: List[Param] = []

    def conv(name, cout, cin, k, region=REGION_DEEP):
        ps.append(Param(name + ".weight", cout * cin * k * k, region))

    def bn(name, c):
        ps.append(Param(name + ".weight", c, REGION_BN_WEIGHT))
        ps.append(Param(name + ".bias", c, REGION_BN_BIAS))

    conv("conv1", 64, 3, 7, REGION_FIRST)
    bn("bn1", 64)
    cin = 64
    for stage, (width, blocks) in enumerate(zip((64, 128, 256, 512), (3, 4, 6, 3))):
        for b in range(blocks):
            pre = f"layer{stage + 1}.{b}"
            conv(pre + ".conv1", width, cin, 1)
            bn(pre + ".bn1", width)
            conv(pre + ".conv2", width, width, 3)
            bn(pre + ".bn2", width)
            conv(pre + ".conv3", width * 4, width, 1)
            bn(pre + ".bn3", width * 4)
            if b == 0:
                conv(pre + ".downsample.0", width * 4, cin, 1)
                bn(pre + ".downsample.1", width * 4)
            cin = width * 4
    ps.append(Param("fc.weight", 1000 * 2048, REGION_FC_WEIGHT))
    ps.append(Param("fc.bias", 1000, REGION_FC_BIAS))
    return ps


def gpt_decoder(n_layer=24, d=2048, ffn=8192, vocab=50257, n_ctx=2048) -> List[Param]:
    """GPT-style decoder (learned positions, biases, tied LM head).
    Defaults: the 1.3B shape, 292 tensors, 1,315,723,264 elements.
    Two-bucket tags: LayerNorm gamma/beta -> BN_WEIGHT/BN_BIAS, token and
    position embeddings -> FIRST, every block linear weight/bias -> DEEP."""
    ps = [Param("wte", vocab * d, REGION_FIRST), Param("wpe", n_ctx * d, REGION_FIRST)]
    for l in range(n_layer):
        pre = f"h.{l}"
        ps += [Param(pre + ".ln_1.weight", d, REGION_BN_WEIGHT),
               Param(pre + ".ln_1.bias", d, REGION_BN_BIAS),
               Param(pre + ".attn.c_attn.weight", d * 3 * d, REGION_DEEP),
               Param(pre + ".attn.c_attn.bias", 3 * d, REGION_DEEP),
               Param(pre + ".attn.c_proj.weight", d * d, REGION_DEEP),
               Param(pre + ".attn.c_proj.bias", d, REGION_DEEP),
               Param(pre + ".ln_2.weight", d, REGION_BN_WEIGHT),
               Param(pre + ".ln_2.bias", d, REGION_BN_BIAS),
               Param(pre + ".mlp.c_fc.weight", d * ffn, REGION_DEEP),
               Param(pre + ".mlp.c_fc.bias", ffn, REGION_DEEP),
               Param(pre + ".mlp.c_proj.weight", ffn * d, REGION_DEEP),
               Param(pre + ".mlp.c_proj.bias", d, REGION_DEEP)]
    ps += [Param("ln_f.weight", d, REGION_BN_WEIGHT), Param("ln_f.bias", d, REGION_BN_BIAS)]
    return ps


def llama(n_layer=32, d=4096, ffn=11008, vocab=32000) -> List[Param]:
    """Llama-style decoder (no biases, RMSNorm, untied LM head).
    Defaults: the 7B shape, 291 tensors, 6,738,415,616 elements."""
    ps = [Param("embed_tokens", vocab * d, REGION_FIRST)]
    for l in range(n_layer):
        pre = f"layers.{l}"
        ps += [Param(pre + ".q_proj", d * d, REGION_DEEP),
               Param(pre + ".k_proj", d * d, REGION_DEEP),
               Param(pre + ".v_proj", d * d, REGION_DEEP),
               Param(pre + ".o_proj", d * d, REGION_DEEP),
               Param(pre + ".gate_proj", ffn * d, REGION_DEEP),
               Param(pre + ".up_proj", ffn * d, REGION_DEEP),
               Param(pre + ".down_proj", d * ffn, REGION_DEEP),
               Param(pre + ".input_layernorm", d, REGION_BN_WEIGHT),
               Param(pre + ".post_attention_layernorm", d, REGION_BN_WEIGHT)]
    ps += [Param("norm", d, REGION_BN_WEIGHT), Param("lm_head", vocab * d, REGION_FC_WEIGHT)]
    return ps


def many_small(n: int = 20000, lo: int = 64, hi: int = 65536, seed: int = 0,
               stream: int = 0x5A11) -> List[Param]:
    """n tensors whose sizes are log-uniform in [lo, hi]:
    u ~ U(ln lo, ln hi), size = clamp(floor(e^u), lo, hi)."""
    u = uniform_f64(seed, stream, n)
    a, b = math.log(lo), math.log(hi)
    sizes = np.floor(np.exp(a + (b - a) * u)).astype(np.int64)
    sizes = np.clip(sizes, lo, hi)
    return [Param(f"t{i}", int(s), REGION_DEEP) for i, s in enumerate(sizes)]


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    n_ranks: int
    params: List[Param]
    dtype: str            # gradient dtype: "f32" or "bf16"
    out_dtype: str        # output dtype
    bucket_cap_bytes: int
    orders: Sequence[str]
    sigma: float
    stream: int           # Philox stream id of the gradient values
    two_bucket: bool = False
    notes: str = ""

    @property
    def numel(self) -> List[int]:
        return [p.numel for p in self.params]

    @property
    def regions(self) -> List[int]:
        return [p.region for p in self.params]

    @property
    def total(self) -> int:
        return sum(p.numel for p in self.params)

    @property
    def in_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def out_bytes(self) -> int:
        return 4 if self.out_dtype == "f32" else 2

    def sync_bytes(self) -> int:
        """Algorithmic bytes of one reduce+scale over all buckets:
        every rank's gradients read once, the average written once."""
        return self.n_ranks * self.total * self.in_bytes + self.total * self.out_bytes


def workload(name: str) -> Workload:
    if name == "tiny":
        return Workload("tiny", 2, tiny_linear(), "f32", "f32", 25 * MiB,
                        ("seq",), 1e-2, 1)
    if name == "resnet50":
        return Workload("resnet50", 8, resnet50(), "f32", "f32", 25 * MiB,
                        ("seq", "ring"), 1e-3, 2)
    if name == "many_small":
        return Workload("many_small", 4, many_small(), "f32", "f32", 1 * MiB,
                        ("ring",), 1e-3, 3)
    if name == "gpt1p3b":
        return Workload("gpt1p3b", 8, gpt_decoder(), "f32", "f32", 25 * MiB,
                        ("ring",), 1e-3, 4)
    if name == "gpt1p3b_two_bucket":
        return Workload("gpt1p3b_two_bucket", 8, gpt_decoder(), "f32", "f32", 25 * MiB,
                        ("ring",), 1e-3, 4, two_bucket=True)
    if name == "llama7b":
        return Workload("llama7b", 8, llama(), "bf16", "bf16", 25 * MiB,
                        ("seq", "ring"), 1e-3, 5)
    raise KeyError(name)


WORKLOADS = ("tiny", "resnet50", "many_small", "gpt1p3b", "gpt1p3b_two_bucket", "llama7b")


def host_rank_flat(wl: Workload, rank: int, base_seed: int = 0,
                   n: Optional[int] = None) -> np.ndarray:
    """Rank ``rank``'s flat gradient buffer on the host (f32 values, or bf16
    bit patterns as uint16 for bf16 workloads).  ``n`` truncates the stream."""
    n = wl.total if n is None else n
    x = normal_f32(base_seed + rank, wl.stream, n, wl.sigma)
    if wl.dtype == "bf16":
        return f32_to_bf16_bits_input(x)
    return x


def device_normal_(t, seed: int, stream: int, sigma: float):
    """Fill a CUDA tensor in place with Normal(0, sigma) values from torch's
    seeded device generator (used for the multi-GB workloads)."""
    import torch
    g = torch.Generator(device=t.device)
    g.manual_seed((seed * 1_000_003 + stream) & ((1 << 63) - 1))
    flat = t.view(-1)
    step = 1 << 30
    for a in range(0, flat.numel(), step):
        flat[a:a + step].normal_(0.0, sigma, generator=g)
    return t
