"""GPU parity of the raw fallback (a plan with ZC_PLAN_RAW_FALLBACK keeps the
smaller of the coded and the raw stream; reading stated in the oracle's C
file): device streams against the oracle's byte for byte on both sides of the
break-even point, decoding of raw streams from buffers longer and shorter than
the coded layout, strict rejection of corrupt raw headers, and raw peers in
the local reduction.  Integer and byte work: the bar is equality."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins
from gpu_util import compress_batch, decompress_batch, require_gpu, to_device, to_host_u16
from lossless_bf16_exponent_amd import workloads

pytestmark = pytest.mark.gpu

WINDOW_PLAN = oracle_pins.WINDOW_PLAN
FILL = 0x2BCD


@pytest.fixture(scope="module")
def zc():
    return require_gpu()


def fb(zc, exps):
    return zc.plan_with_raw_fallback(exps)


def dev(x):
    return to_device(x) if x.size else None


def decode_exact(zc, stream: np.ndarray, n: int, in_bytes=None):
    """Decode a stream copied into a buffer of exactly its size (or in_bytes)."""
    nb = stream.size if in_bytes is None else in_bytes
    m = min(nb, stream.size)
    buf = torch.zeros(max(nb, 128), dtype=torch.uint8, device="cuda")
    buf[:m] = torch.from_numpy(stream[:m].copy()).cuda()
    out = torch.full((max(n, 1),), FILL, dtype=torch.int16, device="cuda")
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    zc.zc_decompress(buf, nb, n, out, st)
    torch.cuda.synchronize()
    return to_host_u16(out[:n]), int(st.item()), to_host_u16(out)


def break_even_cases(n):
    lay = oracle.layout(n)
    T = 128 + 2 * n - lay["off_zp"]
    return sorted({e for e in (0, T - 1, T, T + 1, n) if 0 <= e <= n})


@pytest.mark.parametrize("n", [1, 7, 100, 1000, 4096, 10_000, 65_539, 1_000_003])
def test_fallback_streams_match_oracle(zc, n):
    for E in break_even_cases(n):
        print("fallback n=%d E=%d" % (n, E), flush=True)
        x = oracle_pins.with_escapes(n, E, 7 * n + E)
        enc = compress_batch(zc, [dev(x)], [n], [fb(zc, WINDOW_PLAN)])
        ref = oracle.encode(x, WINDOW_PLAN, raw_fallback=True)
        got = enc.stream(0)
        assert got.size == ref.size and np.array_equal(got, ref), (n, E)
        assert zc.zc_read_header(got[:128].tobytes())["raw"] == (ref.size == 128 + 2 * n and ref[31] == 1)
        outs, status = decompress_batch(zc, enc, [n])            # from the capacity-sized buffer
        assert not status.any() and np.array_equal(to_host_u16(outs[0][:n]), x)
        y, st, _ = decode_exact(zc, ref, n)                         # from a buffer of exactly total_bytes
        assert st == 0 and np.array_equal(y, x), (n, E)


def test_without_the_flag_streams_stay_coded(zc):
    n = 10_000
    x = oracle_pins.with_escapes(n, n, 3)
    enc = compress_batch(zc, [dev(x)], [n], [WINDOW_PLAN])
    assert np.array_equal(enc.stream(0), oracle.encode(x, WINDOW_PLAN))
    assert enc.stream(0).size > 128 + 2 * n


def test_fallback_mixed_batch(zc):
    """Flagged and plain segments, raw and coded outcomes, empty and tiny
    segments in one launch: each equals the oracle's stream for its plan."""
    specs = [(40_000, 40_000, True), (40_000, 100, True), (40_000, 40_000, False), (0, 0, True),
             (5, 0, True), (70_001, 69_000, True), (8192, 8192, False), (123_457, 30_000, True)]
    xs = [oracle_pins.with_escapes(n, E, 11 + i) for i, (n, E, _) in enumerate(specs)]
    plans = [fb(zc, WINDOW_PLAN) if f else WINDOW_PLAN for (_, _, f) in specs]
    ns = [n for (n, _, _) in specs]
    enc = compress_batch(zc, [dev(x) for x in xs], ns, plans)
    for i, (x, (n, E, f)) in enumerate(zip(xs, specs)):
        ref = oracle.encode(x, WINDOW_PLAN, raw_fallback=f)
        assert np.array_equal(enc.stream(i), ref), i
    outs, status = decompress_batch(zc, enc, ns)
    assert not status.any()
    for o, x, n in zip(outs, xs, ns):
        assert np.array_equal(to_host_u16(o[:n]), x)
    # the same streams in exact-size buffers, some shorter than the coded layout
    segs, bufs, outs2 = [], [], []
    st = torch.full((len(ns),), -1, dtype=torch.int32, device="cuda")
    for i, n in enumerate(ns):
        s = enc.stream(i)
        b = torch.zeros(max(s.size, 128), dtype=torch.uint8, device="cuda")
        b[:s.size] = torch.from_numpy(s).cuda()
        o = torch.full((max(n, 1),), FILL, dtype=torch.int16, device="cuda")
        bufs.append(b)
        outs2.append(o)
        segs.append((b, s.size, n, o, st.data_ptr() + 4 * i))
    assert any(enc.stream(i).size < oracle.layout(n)["off_zp"] for i, n in enumerate(ns))
    zc.zc_decompress_batch(segs)
    torch.cuda.synchronize()
    assert not st.cpu().numpy().any()
    for o, x, n in zip(outs2, xs, ns):
        assert np.array_equal(to_host_u16(o[:n]), x)


@pytest.mark.parametrize("n", [100, 10_000])
def test_corrupt_raw_headers_are_rejected(zc, n):
    """n = 100: the raw stream is shorter than the coded layout (the raw-only
    decode path); n = 10,000: longer (the coded decoder's fallback check)."""
    x = oracle_pins.with_escapes(n, n, 5)
    ref = oracle.encode(x, WINDOW_PLAN, raw_fallback=True)
    assert ref[31] == 1
    y, st, _ = decode_exact(zc, ref, n)
    assert st == 0 and np.array_equal(y, x)
    cases = {"mode 2": (31, 2), "mode 0": (31, 0), "total": (40, ref[40] ^ 2), "pad": (100, 1),
             "magic": (0, ref[0] ^ 1), "E > n": (39, 0x80)}
    for name, (pos, val) in cases.items():
        bad = ref.copy()
        bad[pos] = val
        _, st, whole = decode_exact(zc, bad, n)
        assert st == zc.ZC_ERR_CORRUPT, name
        assert (whole == FILL).all(), name  # nothing written
    # a buffer one byte short of the raw stream
    if ref.size - 1 < oracle.layout(n)["off_zp"]:
        assert zc.raw_status("zc_decompress", 0x7F0000000000, ref.size - 1, n, 0x7F1000000000, 0, 0) \
            == zc.ZC_ERR_CORRUPT
    else:
        _, st, whole = decode_exact(zc, ref, n, in_bytes=ref.size - 1)
        assert st == zc.ZC_ERR_CORRUPT and (whole == FILL).all()


@pytest.mark.parametrize("n", [100, 9000, 100_003])
def test_reduce_with_raw_peers(zc, n):
    """Raw and coded peers in one local reduction, raw ones also in buffers of
    exactly their size, against the oracle's decode_reduce."""
    g = np.random.default_rng(n)
    peers = [workloads.bf16_bits_from_f32((g.standard_normal(n) * 2e-3).astype(np.float32)),
             oracle_pins.with_escapes(n, n, 1),
             oracle_pins.with_escapes(n, n // 2, 2),
             workloads.bf16_bits_from_f32((g.standard_normal(n) * 5e-4).astype(np.float32))]
    local = workloads.bf16_bits_from_f32((g.standard_normal(n) * 1e-3).astype(np.float32))
    plans = [oracle.plan_from_sigma(2e-3), WINDOW_PLAN, WINDOW_PLAN, oracle.plan_from_sigma(5e-4)]
    refs = [oracle.encode(x, p, raw_fallback=True) for x, p in zip(peers, plans)]
    assert refs[1][31] == 1
    enc = compress_batch(zc, [dev(x) for x in peers], [n] * 4, [fb(zc, p) for p in plans])
    for i in range(4):
        assert np.array_equal(enc.stream(i), refs[i]), i
    bufs = []
    for r in refs:
        b = torch.zeros(r.size, dtype=torch.uint8, device="cuda")
        b[:] = torch.from_numpy(r).cuda()
        bufs.append(b)
    out = torch.full((n,), FILL, dtype=torch.int16, device="cuda")
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    zc.zc_decompress_reduce([b.data_ptr() for b in bufs], [r.size for r in refs], n, to_device(local), out, st)
    torch.cuda.synchronize()
    rc, ref = oracle.decode_reduce(refs, n, local)
    assert rc == 0 and int(st.item()) == 0
    assert np.array_equal(to_host_u16(out), ref)


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["5b", "5a"])
def test_full_size_stress_goes_raw(zc, name):
    """The two stress workloads that coding expands (sigma mismatch, uniform
    patterns) come out raw under the fallback, with the oracle's header; the
    payload is the input and decodes back to it."""
    w = workloads.get(name)
    seg = w.segments[0]
    p = zc.zc_plan_from_sigma(seg.sigma)
    n = w.n
    print("fallback full size %s n=%d" % (w.name, n), flush=True)
    d = to_device(w.buffer)
    enc = compress_batch(zc, [d], [n], [fb(zc, p)])
    assert int(enc.totals[0]) == 128 + 2 * n
    o = enc.offsets[0]
    hdr = enc.buf[o:o + 128].cpu().numpy()
    if n <= (1 << 24):
        ref = oracle.encode(w.buffer, p, raw_fallback=True)
        assert np.array_equal(enc.stream(0), ref)
    else:
        hist = oracle.exponent_histogram(w.buffer)
        E = n - int(hist[list(p)].sum())
        ref_hdr = oracle.encode(np.zeros(0, np.uint16), p)[:128].copy()  # the fields that do not depend on the data
        assert bytes(hdr[0:8]) == bytes(ref_hdr[0:8]) and bytes(hdr[16:20]) == bytes(ref_hdr[16:20])
        assert int.from_bytes(hdr[20:24].tobytes(), "little") == oracle.layout(n)["groups"]
        assert int.from_bytes(hdr[8:16].tobytes(), "little") == n
        assert tuple(hdr[24:31]) == tuple(p) and hdr[31] == 1
        assert int.from_bytes(hdr[32:40].tobytes(), "little") == E
        assert oracle.layout(n)["off_zp"] + E > 128 + 2 * n
    assert torch.equal(enc.buf[o + 128:o + 128 + 2 * n].view(torch.int16), d)
    outs, status = decompress_batch(zc, enc, [n])
    assert not status.any() and torch.equal(outs[0][:n], d)
    del enc, outs, d
    torch.cuda.empty_cache()
