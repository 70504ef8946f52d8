"""The raw fallback's guess.  Under ZC_PLAN_RAW_FALLBACK the first compress
launch guesses, per flagged segment, whether the stream will come out raw,
and writes the raw payload or the coded sections accordingly; the exact rule
(the zero-point count against the break-even count) then decides, and a
second launch completes a wrong guess.  The stream must never depend on the
guess: every case here is compared with the oracle byte for byte.

Two test builds fix the guess for every flagged segment (always raw, always
coded), so both outcomes of both guesses are reached on small inputs, in
direct launches (at most 2048 spans) and staged ones.  The shipped build
samples 1024 chunks of 8 values spread evenly over a segment of at least 64
spans; inputs whose escapes avoid, or fill, exactly the sampled chunks make
it guess wrong both ways."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins
from gpu_util import compress_batch, decompress_batch, load_test_build, require_gpu, to_device, to_host_u16
from lossless_bf16_exponent_amd import _build

pytestmark = pytest.mark.gpu

WINDOW_PLAN = oracle_pins.WINDOW_PLAN
SPAN = 8192


@pytest.fixture(scope="module")
def zc():
    return require_gpu()


@pytest.fixture(scope="module", params=["raw", "coded"])
def guess(request, zc):
    return request.param, load_test_build(zc, _build.GUESS_LIBS[request.param])


def break_even(n):
    return 128 + 2 * n - oracle.layout(n)["off_zp"]  # raw iff E > this


def check_batch(zc, specs, lib=None, seed=0, workspace=False):
    """specs: (n, E, flagged) per segment; compress in one call (workspace: the
    _ws call), compare every stream with the oracle's and decode every one back."""
    xs = [oracle_pins.with_escapes(n, E, seed + 31 * i) for i, (n, E, _) in enumerate(specs)]
    ns = [n for (n, _, _) in specs]
    plans = [zc.plan_with_raw_fallback(WINDOW_PLAN) if f else WINDOW_PLAN for (_, _, f) in specs]
    devs = [to_device(x) if x.size else None for x in xs]
    enc = compress_batch(zc, devs, ns, plans, lib=lib, workspace=workspace)
    for i, (x, (n, E, f)) in enumerate(zip(xs, specs)):
        ref = oracle.encode(x, WINDOW_PLAN, raw_fallback=f)
        got = enc.stream(i)
        assert got.size == ref.size and np.array_equal(got, ref), (i, n, E, f)
    outs, status = decompress_batch(zc, enc, ns)
    assert not status.any()
    for o, x, n in zip(outs, xs, ns):
        assert np.array_equal(to_host_u16(o[:n]), x)
    return enc


def direct_specs():
    specs = []
    for n in (1, 100, 8191, 3 * SPAN + 5, 70_001, 40 * SPAN + 3):
        T = break_even(n)
        for E in sorted({e for e in (0, T - 1, T, T + 1, n) if 0 <= e <= n}):
            specs.append((n, E, True))
    specs += [(0, 0, True), (5000, 5000, False), (SPAN, 0, False)]
    return specs


def test_forced_guess_direct_launch(zc, guess):
    """Every break-even case of several sizes, flagged, in launches of at most
    2048 spans (direct placement), both outcomes under the forced guess; every
    other batch through a workspace."""
    name, lib = guess
    specs = direct_specs()
    for lo in range(0, len(specs), 16):
        part = specs[lo:lo + 16]
        assert sum(-(-n // SPAN) for (n, _, _) in part) <= 2048
        ws = (lo // 16) % 2 == 1
        print("guess %s direct segments %d..%d workspace=%s" % (name, lo, lo + len(part), ws), flush=True)
        check_batch(zc, part, lib=lib, seed=lo, workspace=ws)


@pytest.mark.parametrize("workspace", [False, True], ids=["in-buffer", "workspace"])
def test_forced_guess_staged_launch(zc, guess, workspace):
    """A launch of more than 2048 spans (staged placement): a long flagged
    segment on each side of break-even, short flagged and plain ones; the
    scratch behind each stream, or in a workspace (both launches of the call
    then use it)."""
    name, lib = guess
    n_big = 1200 * SPAN + 77
    T = break_even(n_big)
    specs = [(n_big, T + 1, True), (n_big, T, True), (70_001, 70_001, True), (70_001, 10, True), (100, 100, True),
             (9000, 9000, False), (0, 0, True)]
    print("guess %s staged workspace=%s" % (name, workspace), flush=True)
    check_batch(zc, specs, lib=lib, seed=7, workspace=workspace)


def test_forced_guess_repeated_calls_same_buffers(zc, guess):
    """Two calls into the same buffers, the outcome flipped between them:
    words the first call left in the scratch never pass for the second's."""
    name, lib = guess
    n = 70_001
    T = break_even(n)
    for E, seed in ((T + 1, 1), (T, 2), (n, 3), (0, 4)):
        x = oracle_pins.with_escapes(n, E, seed)
        ref = oracle.encode(x, WINDOW_PLAN, raw_fallback=True)
        if E == T + 1:
            buf = torch.full((zc.zc_compress_capacity(n),), 0x33, dtype=torch.uint8, device="cuda")
            size = torch.zeros(1, dtype=torch.int64, device="cuda")
            d = to_device(x)
        else:
            d.copy_(to_device(x))
        arr, k = zc.make_enc_segs([(d, n, zc.plan_with_raw_fallback(WINDOW_PLAN), buf, buf.numel(), size)])
        assert lib.zc_compress_batch(arr, k, torch.cuda.current_stream().cuda_stream) == zc.ZC_OK
        torch.cuda.synchronize()
        assert int(size.item()) == ref.size, (name, E)
        assert np.array_equal(buf[:ref.size].cpu().numpy(), ref), (name, E)


def sampled_values(n):
    """Positions of the values the shipped build's guess samples in a segment
    of n values (n of at least 64 spans): chunk j*(n/8)/1024 of 8 values, j < 1024."""
    chunks = n // 8
    j = np.arange(1024, dtype=np.int64)
    starts = 8 * (j * chunks // 1024)
    return (starts[:, None] + np.arange(8)).ravel()


def escapes_at(n, where, seed):
    """n patterns inside WINDOW_PLAN except at positions `where` (escapes there)."""
    g = np.random.default_rng(seed)
    e = g.integers(116, 123, n)
    esc = g.integers(0, 249, where.size)
    e[where] = np.where(esc >= 116, esc + 7, esc)
    return ((g.integers(0, 2, n) << 15) | (e << 7) | g.integers(0, 128, n)).astype(np.uint16)


@pytest.mark.parametrize("spans", [100, 2500])
def test_sampled_guess_wrong_both_ways(zc, spans):
    """The shipped build: escapes everywhere but the sampled chunks (it guesses
    coded, the stream is raw), and escapes only in the sampled chunks (it
    guesses raw, the stream is coded); 100 spans is a direct launch, 2500 a
    staged one."""
    n = spans * SPAN + 13
    s = sampled_values(n)
    mask = np.ones(n, bool)
    mask[s] = False
    cases = {"raw outcome": np.nonzero(mask)[0], "coded outcome": s}
    for name, where in cases.items():
        print("sampled guess %s spans=%d" % (name, spans), flush=True)
        x = escapes_at(n, where, spans)
        p = zc.plan_with_raw_fallback(WINDOW_PLAN)
        enc = compress_batch(zc, [to_device(x)], [n], [p])
        ref = oracle.encode(x, WINDOW_PLAN, raw_fallback=True)
        assert (ref[31] == 1) == (name == "raw outcome")
        assert np.array_equal(enc.stream(0), ref), name
        outs, status = decompress_batch(zc, enc, [n])
        assert not status.any() and np.array_equal(to_host_u16(outs[0][:n]), x)
