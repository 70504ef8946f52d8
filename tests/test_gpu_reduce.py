"""GPU parity of the local reduction of the reduce-scatter path (section 2.D):
zc_decompress_reduce (HIP, through the C ABI) against the CPU oracle's
decode_reduce, which gets its own encodings of the same inputs.  Integer
patterns out of a fixed float32 arithmetic, so the bar is bit equality."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins
from gpu_util import compress_batch, require_gpu, to_device, to_host_u16
from lossless_bf16_exponent_amd import workloads

pytestmark = pytest.mark.gpu

WINDOW_PLAN = (116, 117, 118, 119, 120, 121, 122)


@pytest.fixture(scope="module")
def zc():
    return require_gpu()


def gaussian(n, sigma, seed):
    g = np.random.default_rng(seed)
    return workloads.bf16_bits_from_f32((g.standard_normal(n) * sigma).astype(np.float32))


def gpu_reduce(zc, peers, plans, local=None, in_place=False, status_fill=-1, streams=None):
    """Compress the peers on the GPU, reduce them on the GPU; returns (out, status)."""
    n = peers[0].size if peers else local.size
    if streams is None:
        enc = compress_batch(zc, [to_device(x) if n else None for x in peers], [n] * len(peers), plans) if peers else None
        ptrs = [enc.buf.data_ptr() + enc.offsets[i] for i in range(len(peers))] if peers else []
        sizes = [int(enc.totals[i]) for i in range(len(peers))] if peers else []
    else:
        enc, (ptrs, sizes) = None, streams
    d_local = to_device(local) if local is not None and n else None
    out = d_local if in_place else torch.full((max(n, 1),), 0x1357, dtype=torch.int16, device="cuda")
    st = torch.full((1,), status_fill, dtype=torch.int32, device="cuda")
    zc.zc_decompress_reduce(ptrs, sizes, n, d_local, out, st)
    torch.cuda.synchronize()
    return to_host_u16(out[:n]), int(st.item()), enc


def oracle_reduce(peers, plans, local=None):
    n = peers[0].size if peers else local.size
    rc, ref = oracle.decode_reduce([oracle.encode(x, p) for x, p in zip(peers, plans)], n, local)
    assert rc == 0
    return ref


@pytest.mark.parametrize("n", [0, 1, 7, 8191, 8192, 8193, 100_003, 1_000_003])
@pytest.mark.parametrize("k", [1, 2, 7])
@pytest.mark.parametrize("with_local", [False, True])
def test_reduce_matches_oracle(zc, n, k, with_local):
    sig = [1e-3, 2e-3, 5e-4, 1e-2, 3e-3, 1e-3, 7e-3, 2e-3]
    peers = [gaussian(n, sig[i], 1000 * k + i + n) for i in range(k)]
    plans = [oracle.plan_from_sigma(s) for s in sig[:k]]
    local = gaussian(n, 4e-3, n + 77) if with_local else None
    got, status, _ = gpu_reduce(zc, peers, plans, local)
    assert status == 0
    assert np.array_equal(got, oracle_reduce(peers, plans, local))


def test_reduce_all_bit_patterns(zc):
    """NaN payloads, infinities, signed zeros, subnormals in every peer."""
    peers = [oracle_pins.all_patterns(seed=s) for s in (1, 2, 3)]
    plans = [WINDOW_PLAN, oracle_pins.HAND_PLAN, (0, 1, 2, 3, 4, 5, 6)]
    local = oracle_pins.all_patterns(seed=4)
    got, status, _ = gpu_reduce(zc, peers, plans, local)
    assert status == 0
    assert np.array_equal(got, oracle_reduce(peers, plans, local))


def test_reduce_local_only_and_in_place(zc):
    n = 70_001
    local = gaussian(n, 0.02, 5)
    got, status, _ = gpu_reduce(zc, [], [], local)          # k = 0: the local share, rounded (identity)
    assert status == 0 and np.array_equal(got, local)
    peers = [gaussian(n, 0.01, 6), gaussian(n, 0.03, 7)]
    got, status, _ = gpu_reduce(zc, peers, [WINDOW_PLAN] * 2, local, in_place=True)
    assert status == 0 and np.array_equal(got, oracle_reduce(peers, [WINDOW_PLAN] * 2, local))


def test_reduce_max_batch(zc):
    n = 9_000
    peers = [gaussian(n, 0.02 * (1 + i % 5), 50 + i) for i in range(64)]
    got, status, _ = gpu_reduce(zc, peers, [WINDOW_PLAN] * 64)
    assert status == 0 and np.array_equal(got, oracle_reduce(peers, [WINDOW_PLAN] * 64))


def test_reduce_rejects_bad_stream_and_writes_nothing(zc):
    n = 30_000
    peers = [gaussian(n, 0.02, 8), gaussian(n, 0.02, 9)]
    streams = [oracle.encode(x, WINDOW_PLAN) for x in peers]
    bad = streams[1].copy()
    bad[8] ^= 0x01                                            # header n
    bufs = [torch.from_numpy(np.concatenate([s, np.zeros(256, np.uint8)])).cuda() for s in (streams[0], bad)]
    got, status, _ = gpu_reduce(zc, peers, None, streams=([b.data_ptr() for b in bufs], [s.size for s in streams]))
    assert status == 4 and bool((got == 0x1357).all())
    # a table entry off by one: caught per 4096-value group
    lay = oracle.layout(n)
    bad = streams[1].copy()
    bad[lay["off_tab"] + 4] ^= 0x01
    bufs = [torch.from_numpy(np.concatenate([s, np.zeros(256, np.uint8)])).cuda() for s in (streams[0], bad)]
    _, status, _ = gpu_reduce(zc, peers, None, streams=([b.data_ptr() for b in bufs], [s.size for s in streams]))
    assert status == 4


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_reduce_full_shard(zc):
    """The reduce-scatter share of the 256M gradient bucket on 8 GPUs: 32M
    values from 7 peers (each with its own sigma plan) plus the local share."""
    n = 1 << 25
    sig = workloads.config3_sigmas()[:8]
    xs = [gaussian(n, float(s), 9000 + i) for i, s in enumerate(sig)]
    plans = [oracle.plan_from_sigma(float(s)) for s in sig[1:]]
    print("full shard: n=%d, 7 peers + local" % n, flush=True)
    got, status, _ = gpu_reduce(zc, xs[1:], plans, xs[0])
    assert status == 0
    assert np.array_equal(got, oracle_reduce(xs[1:], plans, xs[0]))


def half_escapes(n, counts, seed):
    """WINDOW_PLAN-coded patterns where the 2048-value half h of every tile holds
    counts[h % len(counts)] zero-points (fewer if the half is shorter)."""
    g = np.random.default_rng(seed)
    e = g.integers(116, 123, n)
    for h, v0 in enumerate(range(0, n, 2048)):
        m = min(2048, n - v0)
        c = min(counts[h % len(counts)], m)
        idx = v0 + g.choice(m, c, replace=False)
        esc = g.integers(0, 249, c)
        e[idx] = np.where(esc >= 116, esc + 7, esc)
    return ((g.integers(0, 2, n) << 15) | (e << 7) | g.integers(0, 128, n)).astype(np.uint16)


@pytest.mark.parametrize("n", [4096 * 3 + 2049, 4096 * 4, 2048 + 17])
def test_reduce_many_zero_points_per_half(zc, n):
    """Halves with more zero-points than a wave stages (more than 1024) read
    them another way; exactly 1024 still fits.  Mixed with an ordinary peer, a
    half-filled last tile and the local share."""
    cycles = [[0, 1024, 1025, 2048, 300, 1500], [1024, 0, 2048, 1025, 1500, 300], [2048, 2048, 1, 1024]]
    peers = [half_escapes(n, c, 300 + i) for i, c in enumerate(cycles)] + [gaussian(n, 3e-3, 31)]
    plans = [WINDOW_PLAN] * 3 + [oracle.plan_from_sigma(3e-3)]
    local = gaussian(n, 1e-3, 32)
    got, status, _ = gpu_reduce(zc, peers, plans, local)
    assert status == 0
    assert np.array_equal(got, oracle_reduce(peers, plans, local))


@pytest.mark.parametrize("v", [4096 + 5, 4096 + 2048 + 1000, 3 * 4096 + 2047])
def test_reduce_plane_count_mismatch_is_caught(zc, v):
    """A value's code turned into the zero-point code (its three plane bits
    cleared) changes its half's zero-point count against the table: the two
    halves of the tile then disagree on where one's zero-points end and the
    other's begin, and the status says so."""
    n = 30_000
    x = gaussian(n, 0.02, 40)
    lay = oracle.layout(n)
    s = oracle.encode(x, WINDOW_PLAN)
    bits = [(s[lay["off_p%d" % p] + v // 8] >> (v % 8)) & 1 for p in range(3)]
    assert any(bits), "value %d already a zero-point" % v
    bad = s.copy()
    for p in range(3):
        bad[lay["off_p%d" % p] + v // 8] &= ~np.uint8(1 << (v % 8))
    good = oracle.encode(gaussian(n, 0.01, 41), WINDOW_PLAN)
    bufs = [torch.from_numpy(np.concatenate([b, np.zeros(256, np.uint8)])).cuda() for b in (good, bad)]
    _, status, _ = gpu_reduce(zc, [x, x], None, streams=([b.data_ptr() for b in bufs], [good.size, bad.size]))
    assert status == 4
