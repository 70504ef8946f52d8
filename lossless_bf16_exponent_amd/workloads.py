"""Seeded synthetic BF16 inputs shaped like the workloads on the ZipCCL pages.

This module only draws numbers and rounds them to BF16; it holds none of the
codec's arithmetic (no exponent split, no table, no codes), so that the CPU
oracle and the HIP library can both be fed from it.

The pages evaluate on Llama3-8B (all-gather of dense parameters), Qwen3-MoE and
DeepSeek-V3 (MoE all-to-all) training traffic ("Experimental results" section
of the explainer).  No weights, activations or datasets are available here, so
every input is drawn from the distribution family the pages name for training
tensors -- near-Gaussian (section 2.A) -- with the shapes of those workloads:

  1  1,048,576 values of N(0, 0.02^2); plan from sigma = 0.02
  2  one 4096 x 14336 Llama3-8B-shaped parameter shard, N(0, 0.02^2)
  3  a 256 Mi-element gradient bucket of 32 layer segments, per-segment sigma
     log-uniform in [1e-5, 1e-2], 1 % exact zeros per segment
  4  MoE all-to-all payload: 8192 tokens x top-8 routing x hidden 7168, Student-t
     (nu = 5) values scaled to unit variance; per destination one static
     (equal-size) and one dynamic (Zipf(1.2) expert-load) segment
  5a 2^30 values of N(0, 0.16^2) coded with the sigma = 0.02 plan
  5b 16 Mi uniformly random 16-bit patterns excluding NaN/Inf, sigma = 0.02 plan

BF16 values are float32 draws rounded to nearest-even, the conversion a
framework applies when it casts float32 to bfloat16.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK = 1 << 24  # elements drawn per generator stream for the large buffers


def _parallel(fn, items) -> None:
    """fn(item) for every item, on a few threads.  Each item draws from its own
    seeded generator into its own slice, so the result does not depend on the
    order or the thread count (numpy's generators release the GIL while they
    fill an array)."""
    items = list(items)
    workers = max(1, min(len(items), 8, len(os.sched_getaffinity(0))))
    if workers == 1:
        for it in items:
            fn(it)
        return
    with ThreadPoolExecutor(workers) as ex:
        for _ in ex.map(fn, items):
            pass


def bf16_bits_from_f32(f: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 patterns.

    Inputs here are finite; NaN payload handling is not needed."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
    return r.astype(np.uint16)


@dataclass
class Segment:
    name: str
    x: np.ndarray  # uint16 BF16 patterns (a view into Workload.buffer)
    sigma: float  # the sigma the segment's exponent table is built from


@dataclass
class Workload:
    name: str
    description: str
    buffer: np.ndarray  # all segments back to back, uint16
    segments: list = field(default_factory=list)

    @property
    def n(self) -> int:
        return int(self.buffer.size)


def _normal_blocks(out: np.ndarray, key: int, sigma: float) -> None:
    """out[:] = bf16(N(0,1) * sigma) drawn block by block with seeds [key, b]."""
    s = np.float32(sigma)

    def block(b):
        start = b * BLOCK
        m = min(BLOCK, out.size - start)
        g = np.random.default_rng([key, b])
        out[start:start + m] = bf16_bits_from_f32(g.standard_normal(m, dtype=np.float32) * s)

    _parallel(block, range((out.size + BLOCK - 1) // BLOCK))


def config1() -> Workload:
    n = 1 << 20
    f = np.random.default_rng(0).standard_normal(n, dtype=np.float32) * np.float32(0.02)
    buf = bf16_bits_from_f32(f)
    return Workload("single-tensor-1M", "1,048,576 x N(0, 0.02^2), one stream", buf,
                    [Segment("tensor", buf, 0.02)])


def config2() -> Workload:
    n = 4096 * 14336
    buf = np.empty(n, dtype=np.uint16)
    _normal_blocks(buf, 1, 0.02)
    return Workload("llama3-8b-allgather-shard-4096x14336",
                    "Llama3-8B-shaped 4096 x 14336 parameter shard, N(0, 0.02^2), one stream", buf,
                    [Segment("shard", buf, 0.02)])


CONFIG3_SEGMENTS = 32
CONFIG3_SEG_ELEMS = 8_388_608
CONFIG3_ZEROS = 83_886  # 1 % of each segment


def config3_sigmas() -> np.ndarray:
    return 10.0 ** np.random.default_rng(2).uniform(-5.0, -2.0, CONFIG3_SEGMENTS)


def config3(segments: int = CONFIG3_SEGMENTS) -> Workload:
    sig = config3_sigmas()
    buf = np.empty(segments * CONFIG3_SEG_ELEMS, dtype=np.uint16)

    def segment(s):
        g = np.random.default_rng([2, s])
        v = g.standard_normal(CONFIG3_SEG_ELEMS, dtype=np.float32) * np.float32(sig[s])
        view = buf[s * CONFIG3_SEG_ELEMS:(s + 1) * CONFIG3_SEG_ELEMS]
        view[:] = bf16_bits_from_f32(v)
        view[g.choice(CONFIG3_SEG_ELEMS, CONFIG3_ZEROS, replace=False)] = 0  # +0.0

    _parallel(segment, range(segments))
    segs = [Segment("layer%02d" % s, buf[s * CONFIG3_SEG_ELEMS:(s + 1) * CONFIG3_SEG_ELEMS], float(sig[s]))
            for s in range(segments)]
    return Workload("gradient-bucket-256M-32seg",
                    "256 Mi-element gradient bucket, 32 layer segments, sigma log-uniform "
                    "[1e-5, 1e-2], 1% zeros, per-segment plan", buf, segs)


MOE_TOKENS = 8192
MOE_TOPK = 8
MOE_HIDDEN = 7168
MOE_EXPERTS = 256
MOE_DESTS = 8


def moe_destination_loads() -> np.ndarray:
    """Token-copies per destination rank: Zipf(1.2) popularity over 256 experts,
    32 experts per destination, largest-remainder rounding of T*w/sum(w)."""
    total = MOE_TOKENS * MOE_TOPK
    rank = np.random.default_rng(3).permutation(MOE_EXPERTS) + 1
    w = rank.astype(np.float64) ** -1.2
    share = total * w / w.sum()
    base = np.floor(share).astype(np.int64)
    rest = total - int(base.sum())
    order = np.argsort(-(share - base), kind="stable")
    base[order[:rest]] += 1
    return base.reshape(MOE_DESTS, MOE_EXPERTS // MOE_DESTS).sum(axis=1)


def config4() -> Workload:
    loads = moe_destination_loads()
    static_tokens = int(loads.min())
    sizes = [static_tokens * MOE_HIDDEN] * MOE_DESTS + [int(l - static_tokens) * MOE_HIDDEN for l in loads]
    buf = np.empty(sum(sizes), dtype=np.uint16)
    scale = np.float32(np.sqrt(0.6))  # Student-t(5) has variance 5/3
    starts = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)

    def segment(j):
        m = sizes[j]
        if m:
            t = np.random.default_rng([3, j]).standard_t(5, m).astype(np.float32) * scale
            buf[starts[j]:starts[j] + m] = bf16_bits_from_f32(t)

    _parallel(segment, range(len(sizes)))
    segs = [Segment("%s-dest%d" % ("static" if j < MOE_DESTS else "dynamic", j % MOE_DESTS),
                    buf[starts[j]:starts[j] + sizes[j]], 1.0) for j in range(len(sizes))]
    return Workload("moe-a2a-8192tok-top8-h7168",
                    "MoE all-to-all payload, Student-t(5) at unit variance, 8 static + 8 dynamic "
                    "per-destination segments (one dynamic segment is empty)", buf, segs)


def config5a() -> Workload:
    n = 1 << 30
    buf = np.empty(n, dtype=np.uint16)
    _normal_blocks(buf, 4, 0.16)
    return Workload("stress-1G-sigma-mismatch", "2^30 x N(0, 0.16^2) coded with the sigma=0.02 plan",
                    buf, [Segment("tensor", buf, 0.02)])


def config5b() -> Workload:
    n = 1 << 24
    v = np.random.default_rng(5).integers(0, 65280, n)
    x = (((v >> 7) & 1) << 15) | ((v >> 8) << 7) | (v & 0x7F)
    buf = x.astype(np.uint16)
    return Workload("stress-16M-uniform-patterns",
                    "2^24 uniformly random non-NaN/Inf BF16 patterns, sigma=0.02 plan", buf,
                    [Segment("tensor", buf, 0.02)])


CONFIGS = {"1": config1, "2": config2, "3": config3, "4": config4, "5a": config5a, "5b": config5b}


def get(name: str) -> Workload:
    return CONFIGS[str(name)]()
