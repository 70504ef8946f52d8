"""Seeded random cases against the oracle, to reach combinations the listed
cases do not: batches of segments with sizes at and around the tiling's edges
(64-value plane words, 4096-value groups, 8192-value spans) and at random,
random exponent tables (contiguous or not), zero-point densities from none to
all, the raw-fallback flag per segment, scratch behind the stream or in a
workspace, one batched call or one call per segment, launches placed directly
(at most 2048 spans) or staged; and local reductions over random sets of coded
and raw peers.  Every stream is compared with the oracle's byte for byte and
decoded back; every reduction bit for bit.  Byte and integer work: the bar is
equality."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import compress_batch, decompress_batch, require_gpu, to_device, to_host_u16

pytestmark = pytest.mark.gpu

SPAN = 8192
EDGES = [1, 2, 63, 64, 65, 4095, 4096, 4097, 8191, 8192, 8193, 12_288, 16_383, 16_384, 16_385]


@pytest.fixture(scope="module")
def zc():
    return require_gpu()


def random_plan(g) -> tuple:
    """Seven distinct ascending exponent fields: a window of seven, or seven
    drawn from all 256."""
    if g.random() < 0.5:
        lo = int(g.integers(0, 250))
        return tuple(range(lo, lo + 7))
    return tuple(int(e) for e in np.sort(g.choice(256, 7, replace=False)))


def random_values(g, n: int, exps: tuple, q: float) -> np.ndarray:
    """n BF16 patterns: each exponent field from the table with probability
    1 - q, else any of the 256 (which may still be in the table); random signs
    and mantissas (NaN and infinity patterns included when field 255 comes up)."""
    e = np.where(g.random(n) < q, g.integers(0, 256, n), np.asarray(exps)[g.integers(0, 7, n)])
    return ((g.integers(0, 2, n) << 15) | (e << 7) | g.integers(0, 128, n)).astype(np.uint16)


def random_size(g, big: bool) -> int:
    if big:  # one segment that alone makes the launch staged (over 2048 spans)
        return int(2049 * SPAN + g.integers(-SPAN // 2, 300 * SPAN))
    r = g.random()
    if r < 0.1:
        return 0
    if r < 0.5:
        return int(g.choice(EDGES))
    if r < 0.75:
        return int(SPAN * g.integers(1, 40) + g.integers(-2, 3))
    return int(g.integers(1, 400_000))


@pytest.mark.parametrize("case", range(192))
def test_random_batches(zc, case):
    g = np.random.default_rng(9000 + case)
    big = case % 6 == 5
    k = int(g.integers(1, 7))
    ns = [random_size(g, big and i == 0) for i in range(k)]
    plans = [random_plan(g) for _ in range(k)]
    qs = [float(g.choice([0.0, 0.001, 0.03, 0.3, 0.9, 1.0])) for _ in range(k)]
    flags = [bool(g.random() < 0.35) for _ in range(k)]
    workspace = bool(g.random() < 0.5)
    batch = bool(g.random() < 0.8)
    print("random case %d: n=%s q=%s raw-fallback=%s workspace=%s batch=%s" % (case, ns, qs, flags, workspace, batch),
          flush=True)
    xs = [random_values(g, n, p, q) for n, p, q in zip(ns, plans, qs)]
    dev_plans = [zc.plan_with_raw_fallback(p) if f else p for p, f in zip(plans, flags)]
    enc = compress_batch(zc, [to_device(x) if x.size else None for x in xs], ns, dev_plans, batch=batch,
                         workspace=workspace)
    for i, (x, p, f) in enumerate(zip(xs, plans, flags)):
        ref = oracle.encode(x, p, raw_fallback=f)
        got = enc.stream(i)
        assert got.size == ref.size and np.array_equal(got, ref), (case, i, ns[i])
    outs, status = decompress_batch(zc, enc, ns)
    assert not status.any()
    for o, x, n in zip(outs, xs, ns):
        assert np.array_equal(to_host_u16(o[:n]), x)


@pytest.mark.parametrize("case", range(64))
def test_random_reductions(zc, case):
    g = np.random.default_rng(7000 + case)
    k = int(g.integers(0, 9))
    n = int(g.choice(EDGES)) if g.random() < 0.4 else int(g.integers(1, 300_000))
    with_local = k == 0 or g.random() < 0.6
    in_place = with_local and g.random() < 0.3
    plans = [random_plan(g) for _ in range(k)]
    qs = [float(g.choice([0.0, 0.01, 0.2, 1.0])) for _ in range(k)]
    flags = [bool(g.random() < 0.5) for _ in range(k)]
    print("random reduction %d: k=%d n=%d local=%s in_place=%s q=%s raw-fallback=%s"
          % (case, k, n, with_local, in_place, qs, flags), flush=True)
    peers = [random_values(g, n, p, q) for p, q in zip(plans, qs)]
    local = random_values(g, n, random_plan(g), 0.05) if with_local else None
    refs = [oracle.encode(x, p, raw_fallback=f) for x, p, f in zip(peers, plans, flags)]
    rc, want = oracle.decode_reduce(refs, n, local)
    assert rc == 0
    ptrs, sizes = [], []
    if k:
        dev_plans = [zc.plan_with_raw_fallback(p) if f else p for p, f in zip(plans, flags)]
        enc = compress_batch(zc, [to_device(x) for x in peers], [n] * k, dev_plans)
        for i in range(k):
            assert np.array_equal(enc.stream(i), refs[i]), (case, i)
        ptrs = [enc.buf.data_ptr() + enc.offsets[i] for i in range(k)]
        sizes = [int(enc.totals[i]) for i in range(k)]
    d_local = to_device(local) if with_local else None
    out = d_local if in_place else torch.full((n,), 0x1357, dtype=torch.int16, device="cuda")
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    zc.zc_decompress_reduce(ptrs, sizes, n, d_local, out, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(to_host_u16(out[:n]), want)
