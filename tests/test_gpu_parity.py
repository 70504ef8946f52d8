"""GPU parity: the HIP codec (through the C ABI) against the CPU oracle.

Compressed streams must be byte-identical to the oracle's over [0, total_bytes)
and decoding must return the input bit for bit -- integer work, so the bar is
exact equality.  Small cases span several 8192-element tiles and ragged tails;
the full-size workloads run in the launch configuration bench.py times.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins
from gpu_util import compress_batch, decompress_batch, require_gpu, to_device, to_host_u16
from lossless_bf16_exponent_amd import workloads

pytestmark = pytest.mark.gpu

WINDOW_PLAN = (116, 117, 118, 119, 120, 121, 122)
TABLE_PLANS = [oracle_pins.HAND_PLAN, (0, 1, 2, 3, 4, 5, 6), (0, 2, 3, 4, 5, 6, 7), (249, 250, 251, 252, 253, 254, 255)]
EDGE_N = [0, 1, 7, 8, 9, 63, 64, 65, 511, 512, 513, 4095, 4096, 4097, 8191, 8192, 8193, 16383, 16385,
          100_003, 1_000_003]


@pytest.fixture(scope="module")
def zc():
    return require_gpu()


def roundtrip_check(zc, xs, plans, batch=True, workspace=False):
    """Compress + decompress a list of uint16 arrays; compare with the oracle."""
    ns = [x.size for x in xs]
    devs = [to_device(x) if x.size else None for x in xs]
    enc = compress_batch(zc, devs, ns, plans, batch=batch, workspace=workspace)
    for i, (x, p) in enumerate(zip(xs, plans)):
        ref = oracle.encode(x, p)
        got = enc.stream(i)
        assert got.size == ref.size, (i, x.size, p, got.size, ref.size)
        if not np.array_equal(got, ref):
            bad = np.flatnonzero(got != ref)
            raise AssertionError("stream %d (n=%d, plan=%s) differs at %d bytes, first at %d"
                                 % (i, x.size, p, bad.size, bad[0]))
    outs, status = decompress_batch(zc, enc, ns, batch=batch)
    for i, x in enumerate(xs):
        assert status[i] == 0, (i, status[i])
        if x.size:
            assert np.array_equal(to_host_u16(outs[i][:x.size]), x), i
    return enc


def gaussian(n, sigma, seed):
    g = np.random.default_rng(seed)
    return workloads.bf16_bits_from_f32((g.standard_normal(n) * sigma).astype(np.float32))


def test_config1_single_tensor(zc):
    w = workloads.config1()
    plan = zc.zc_plan_from_sigma(0.02)
    assert plan == oracle.plan_from_sigma(0.02) == WINDOW_PLAN
    enc = roundtrip_check(zc, [w.buffer], [plan], batch=False)
    assert int.from_bytes(enc.stream(0)[32:40].tobytes(), "little") == 22_181


@pytest.mark.parametrize("n", EDGE_N)
def test_edge_sizes_window_plan(zc, n):
    roundtrip_check(zc, [gaussian(n, 0.02, n)], [WINDOW_PLAN], batch=False)


@pytest.mark.parametrize("plan", TABLE_PLANS, ids=str)
def test_edge_sizes_table_plans(zc, plan):
    xs = [gaussian(n, 0.02, 7 * n + 1) for n in EDGE_N]
    roundtrip_check(zc, xs[:16], [plan] * 16)
    roundtrip_check(zc, xs[16:], [plan] * (len(EDGE_N) - 16))


@pytest.mark.parametrize("plan", [WINDOW_PLAN, (122, 123, 124, 125, 126, 127, 128),
                                  (248, 249, 250, 251, 252, 253, 254)] + TABLE_PLANS, ids=str)
def test_all_bit_patterns(zc, plan):
    """Every BF16 pattern (NaN payloads, -0, subnormals, Inf), shuffled, plus a
    sorted copy so that whole tiles are all-escape or escape-free."""
    x = oracle_pins.all_patterns(seed=3)
    roundtrip_check(zc, [x, np.arange(65536, dtype=np.uint16)], [plan, plan])


def test_escape_density_sweep(zc):
    """From no zero-points to all zero-points: N(0, s^2) coded with the 0.02 plan."""
    xs = [gaussian(50_000 + 977 * i, s, i) for i, s in enumerate((0.02, 0.03, 0.05, 0.16, 1.0, 100.0))]
    ex = np.array(WINDOW_PLAN, dtype=np.uint16)
    xs.append(((np.random.default_rng(9).choice(ex, 70_000) << 7)
               | np.random.default_rng(10).integers(0, 128, 70_000).astype(np.uint16)).astype(np.uint16))
    roundtrip_check(zc, xs, [WINDOW_PLAN] * len(xs))


def test_batch_equals_single_and_is_deterministic(zc):
    xs = [gaussian(n, s, i) for i, (n, s) in enumerate([(123_457, 0.02), (0, 1.0), (8192 * 3, 1e-3), (77, 0.5),
                                                        (40_000, 3e-5)])]
    plans = [zc.zc_plan_from_sigma(s) for s in (0.02, 1.0, 1e-3, 0.5, 3e-5)]
    plans[3] = oracle_pins.HAND_PLAN
    ns = [x.size for x in xs]
    devs = [to_device(x) if x.size else None for x in xs]
    a = compress_batch(zc, devs, ns, plans, batch=True)
    b = compress_batch(zc, devs, ns, plans, batch=False, fill=0x11)
    c = compress_batch(zc, devs, ns, plans, batch=True, fill=0x77)
    for i in range(len(xs)):
        assert np.array_equal(a.stream(i), b.stream(i))
        assert np.array_equal(a.stream(i), c.stream(i))
        assert np.array_equal(a.stream(i), oracle.encode(xs[i], plans[i]))
    outs, status = decompress_batch(zc, a, ns, batch=False)
    assert not status.any()
    for x, o in zip(xs, outs):
        if x.size:
            assert np.array_equal(to_host_u16(o[:x.size]), x)


def test_max_batch_of_64_segments(zc):
    """The largest batch: 64 segments in one compress launch (128 grid pieces, so
    the block -> piece lookup spans two wave-wide chunks) and one decompress
    launch (64 segment starts), with empty, tiny, ragged and multi-tile
    segments and a mix of plans."""
    sizes = [0, 1, 4097, 8193, 65_536, 300_001, 17, 8192 * 5]
    xs, plans = [], []
    for i in range(64):
        n = sizes[i % len(sizes)]
        sigma = (0.02, 1e-3, 0.5, 3e-5)[i % 4]
        xs.append(gaussian(n, sigma, 1000 + i))
        plans.append(TABLE_PLANS[i % len(TABLE_PLANS)] if i % 5 == 0 else zc.zc_plan_from_sigma(sigma))
    roundtrip_check(zc, xs, plans)


@pytest.mark.parametrize("batch", [True, False], ids=["batch", "single"])
def test_workspace_calls(zc, batch):
    """The _ws calls: output slots of the stream bound only (the sentinel bytes
    right behind each slot stay untouched), the scratch in a workspace that
    starts with random bytes; a direct launch, a staged one (more than 2048
    spans) and one with raw-fallback segments, each equal to the oracle."""
    small = [gaussian(n, sig, 40 + i) for i, (n, sig) in enumerate(((300_007, 0.02), (8192 * 40 + 5, 1e-3),
                                                                     (0, 0.02), (100, 0.16), (1_000_003, 0.16)))]
    plans = [WINDOW_PLAN, oracle.plan_from_sigma(1e-3), WINDOW_PLAN, WINDOW_PLAN, WINDOW_PLAN]
    print("workspace: direct launch, batch=%s" % batch, flush=True)
    roundtrip_check(zc, small, plans, batch=batch, workspace=True)
    big = small + [gaussian(8192 * 2100 + 11, 0.02, 50)]
    print("workspace: staged launch, batch=%s" % batch, flush=True)
    roundtrip_check(zc, big, plans + [WINDOW_PLAN], batch=batch, workspace=True)
    if batch:
        print("workspace: raw fallback", flush=True)
        xs = [oracle_pins.with_escapes(70_001, 70_001, 3), oracle_pins.with_escapes(8192 * 100 + 3, 100, 4),
              oracle_pins.with_escapes(8192 * 100 + 3, 8192 * 100, 5)]
        ns = [x.size for x in xs]
        enc = compress_batch(zc, [to_device(x) for x in xs], ns, [zc.plan_with_raw_fallback(WINDOW_PLAN)] * 3,
                             workspace=True)
        for i, x in enumerate(xs):
            assert np.array_equal(enc.stream(i), oracle.encode(x, WINDOW_PLAN, raw_fallback=True)), i


def test_output_buffer_reuse_and_old_contents(zc):
    """Calls in a row into one output buffer that starts with random bytes: the
    scratch words left behind by earlier calls (or by anything else) must never
    be taken for the current call's.  Sizes give several finalize blocks."""
    from gpu_util import slot
    for n in (300_007, 1_000_003):
        cap = zc.zc_compress_capacity(n)
        g = torch.Generator(device="cuda").manual_seed(n)
        buf = torch.randint(0, 256, (slot(cap),), dtype=torch.uint8, device="cuda", generator=g)
        size = torch.zeros(1, dtype=torch.int64, device="cuda")
        for i, (sigma, plan) in enumerate(((0.02, WINDOW_PLAN), (0.16, WINDOW_PLAN), (0.16, WINDOW_PLAN),
                                           (1e-3, oracle.plan_from_sigma(1e-3)), (0.05, oracle_pins.HAND_PLAN))):
            x = gaussian(n, sigma, 100 + i)
            zc.zc_compress(to_device(x), n, plan, buf, cap, size)
            torch.cuda.synchronize()
            ref = oracle.encode(x, plan)
            assert int(size.item()) == ref.size, (n, i)
            assert np.array_equal(buf[:ref.size].cpu().numpy(), ref), (n, i)


def test_calls_in_flight_on_two_streams(zc):
    """Compress calls on two HIP streams at once (each call has its own token
    and scratch), several rounds with no synchronization between the streams,
    then decodes on both streams: every stream equals the oracle's and every
    decode the input.  Default stream priority on both."""
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    cases = [(2_000_003, 0.02, WINDOW_PLAN), (1_500_001, 1e-3, oracle.plan_from_sigma(1e-3)),
             (700_001, 0.16, WINDOW_PLAN), (3_000_017, 0.05, oracle_pins.HAND_PLAN)]
    xs = [gaussian(n, sig, 300 + i) for i, (n, sig, _) in enumerate(cases)]
    dev = [to_device(x) for x in xs]
    caps = [zc.zc_max_compressed_bytes(n) for n, _, _ in cases]
    bufs = [torch.empty(c, dtype=torch.uint8, device="cuda") for c in caps]
    # one workspace per stream, reused by every call on it
    wsb = max(zc.zc_compress_workspace_bytes(n) for n, _, _ in cases)
    wss = [torch.empty(wsb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    sizes = torch.zeros(len(cases), dtype=torch.int64, device="cuda")
    outs = [torch.empty_like(d) for d in dev]
    st = torch.full((len(cases),), -1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for rnd in range(3):
        for i, (n, _, plan) in enumerate(cases):
            s = sa if i % 2 == 0 else sb
            zc.zc_compress_ws(dev[i], n, plan, bufs[i], caps[i], sizes.data_ptr() + 8 * i, wss[i % 2], wsb, stream=s)
    for i, (n, _, _) in enumerate(cases):
        s = sa if i % 2 == 0 else sb
        zc.zc_decompress(bufs[i], caps[i], n, outs[i], st.data_ptr() + 4 * i, stream=s)
    torch.cuda.synchronize()
    assert not st.cpu().numpy().any()
    for i, (n, _, plan) in enumerate(cases):
        ref = oracle.encode(xs[i], plan)
        assert int(sizes[i].item()) == ref.size, i
        assert np.array_equal(bufs[i][:ref.size].cpu().numpy(), ref), i
        assert torch.equal(outs[i], dev[i]), i


def test_decoder_reads_oracle_streams(zc):
    """The GPU decoder on streams written by the oracle (not by the GPU encoder)."""
    for n, plan in ((1_000_003, WINDOW_PLAN), (9000, oracle_pins.HAND_PLAN), (0, WINDOW_PLAN)):
        x = gaussian(n, 0.05, n)
        s = oracle.encode(x, plan)
        cap = ((s.size + 255) // 256) * 256
        buf = torch.zeros(cap, dtype=torch.uint8, device="cuda")
        buf[:s.size] = torch.from_numpy(s).cuda()
        out = torch.zeros(max(n, 1), dtype=torch.int16, device="cuda")
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        zc.zc_decompress(buf, s.size, n, out, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert np.array_equal(to_host_u16(out[:n]), x)


def test_decoder_rejects_bad_header_and_writes_nothing(zc):
    n = 30_000
    x = gaussian(n, 0.02, 5)
    s = oracle.encode(x, WINDOW_PLAN)
    lay = oracle.layout(n)
    for pos in (0, 4, 6, 8, 12, 16, 20, 25, 31, 32, 40, 64, 127):
        bad = s.copy()
        bad[pos] ^= 0x40
        buf = torch.from_numpy(np.concatenate([bad, np.zeros(256, np.uint8)])).cuda()
        out = torch.full((n,), 0x1234, dtype=torch.int16, device="cuda")
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        zc.zc_decompress(buf, s.size, n, out, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 4, pos
        assert bool((out == 0x1234).all()), pos
    # wrong n from the caller, and a stream cut short
    buf = torch.from_numpy(np.concatenate([s, np.zeros(256, np.uint8)])).cuda()
    for nn, nbytes in ((n - 1, s.size), (n, s.size - 1)):
        out = torch.full((n,), 0x1234, dtype=torch.int16, device="cuda")
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        if nbytes < lay["off_zp"]:
            continue
        zc.zc_decompress(buf, nbytes, nn, out, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 4
        assert bool((out == 0x1234).all())


def test_decoder_flags_table_corruption(zc):
    n = 50_000
    x = gaussian(n, 0.05, 6)
    s = oracle.encode(x, WINDOW_PLAN)
    lay = oracle.layout(n)
    # a plane bit of a zero-point value: its code turns nonzero and the group's
    # count no longer matches the table (a flip between two nonzero codes is
    # undetectable by any decoder and is not tested)
    zp_index = int(np.flatnonzero(~np.isin(oracle_pins.exponent_field(x), WINDOW_PLAN))[10])
    plane_pos = lay["off_p0"] + zp_index // 8
    for delta_pos, bit in ((lay["off_tab"] + 4, 0x01), (lay["off_tab"] + 12, 0x01), (lay["off_tab"] + 8, 0x02),
                           (plane_pos, 1 << (zp_index % 8))):
        bad = s.copy()
        bad[delta_pos] ^= bit
        buf = torch.from_numpy(np.concatenate([bad, np.zeros(256, np.uint8)])).cuda()
        out = torch.zeros(n, dtype=torch.int16, device="cuda")
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        zc.zc_decompress(buf, s.size, n, out, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 4, delta_pos


def test_stream_size_is_reported(zc):
    x = gaussian(12_345, 0.02, 8)
    enc = compress_batch(zc, [to_device(x)], [x.size], [WINDOW_PLAN], batch=False)
    assert int(enc.totals[0]) == oracle.encode(x, WINDOW_PLAN).size
    info = zc.zc_read_header(enc.stream(0)[:128].tobytes())
    assert info["total_bytes"] == int(enc.totals[0]) and info["n"] == x.size


# ---------------------------------------------------------------------------
# full-size workloads, in the same launch configuration as bench.py
# ---------------------------------------------------------------------------

def full_size_check(zc, w):
    plans = [zc.zc_plan_from_sigma(seg.sigma) for seg in w.segments]
    for seg, p in zip(w.segments, plans):
        assert p == oracle.plan_from_sigma(seg.sigma)
    dev = to_device(w.buffer)
    ns = [seg.x.size for seg in w.segments]
    views, off = [], 0
    for n in ns:
        views.append(dev[off:off + n] if n else None)
        off += n
    print("full-size %s: %d segments, n=%d" % (w.name, len(ns), w.n), flush=True)
    enc = compress_batch(zc, views, ns, plans, batch=True)
    for i, (seg, p) in enumerate(zip(w.segments, plans)):
        ref = oracle.encode(seg.x, p)
        got = enc.stream(i)
        assert got.size == ref.size and np.array_equal(got, ref), (w.name, i)
        del ref, got
    outs, status = decompress_batch(zc, enc, ns, batch=True)
    assert not status.any()
    off = 0
    for n, o in zip(ns, outs):
        if n:
            assert torch.equal(o[:n], dev[off:off + n])
        off += n
    del enc, outs, dev
    torch.cuda.empty_cache()


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["2", "3", "4", "5b", "5a"])
def test_full_size_workload(zc, name):
    full_size_check(zc, workloads.get(name))
