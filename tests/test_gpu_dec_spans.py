"""Both span forms of the decoder on small and ragged inputs.  The shipped
library picks one-tile or two-tile spans by the size of the launch; two test
builds (tests/libzc_dec_narrow.so, tests/libzc_dec_wide.so) take one form for
every launch, so that the cases of the parity tests reach each form: edge
sizes, every bit pattern under several tables, zero-point densities from none
to all, batches of many segments (block ranges of one or two tiles), raw
streams through the coded decoder's raw branch and through the raw-only
decoder, header and table corruption, guard bytes.  Streams come from the
oracle.  Integer and byte work: the bar is equality."""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins
from gpu_util import GUARD, check_untouched, load_test_build, require_gpu, to_host_u16
from lossless_bf16_exponent_amd import _build

pytestmark = pytest.mark.gpu

WINDOW_PLAN = oracle_pins.WINDOW_PLAN
FILL = 0x1234


@pytest.fixture(scope="module")
def zc():
    return require_gpu()


@pytest.fixture(scope="module", params=sorted(_build.SPAN_LIBS))
def lib(zc, request):
    return load_test_build(zc, _build.SPAN_LIBS[request.param])


def decode(zc, lib, streams, ns):
    """Decode oracle streams with the test build in one batched call; each
    stream in its own device buffer (its size rounded up to 256 bytes; in_bytes
    is the stream's exact size), each output with GUARD sentinel bytes on both
    sides.  Returns the outputs (host) and the status words."""
    g = GUARD // 2
    bufs, outs, guards = [], [], []
    for s, n in zip(streams, ns):
        b = torch.zeros(max(128, (s.size + 255) // 256 * 256), dtype=torch.uint8, device="cuda")
        b[:s.size] = torch.from_numpy(s.copy()).cuda()
        bufs.append(b)
        full = torch.full((max(n, 1) + 2 * g,), FILL, dtype=torch.int16, device="cuda")
        guards.append(full)
        outs.append(full[g:g + max(n, 1)])
    st = torch.full((len(ns),), -1, dtype=torch.int32, device="cuda")
    segs = [(b, s.size, n, o, st.data_ptr() + 4 * i) for i, (b, s, n, o) in enumerate(zip(bufs, streams, ns, outs))]
    arr, k = zc.make_dec_segs(segs)
    rc = lib.zc_decompress_batch(arr, k, torch.cuda.current_stream().cuda_stream)
    assert rc == zc.ZC_OK, rc
    torch.cuda.synchronize()
    for full, n in zip(guards, ns):
        check_untouched(full[:g], FILL, "before the output")
        check_untouched(full[g + max(n, 1):], FILL, "after the output")
    return [to_host_u16(o[:n]) for o, n in zip(outs, ns)], st.cpu().numpy()


def gaussian(n, sigma, seed):
    from lossless_bf16_exponent_amd import workloads
    g = np.random.default_rng(seed)
    return workloads.bf16_bits_from_f32((g.standard_normal(n) * sigma).astype(np.float32))


SIZES = [0, 1, 7, 63, 64, 65, 511, 513, 4095, 4096, 4097, 8191, 8192, 8193, 12_289, 16_383, 16_384, 16_385,
         100_003, 1_000_003]


@pytest.mark.parametrize("n", SIZES)
def test_round_trip_edge_sizes(zc, lib, n):
    x = gaussian(n, 0.02, n + 3)
    s = oracle.encode(x, WINDOW_PLAN)
    (y,), st = decode(zc, lib, [s], [n])
    assert st[0] == 0 and np.array_equal(y, x), n


@pytest.mark.parametrize("plan", [WINDOW_PLAN, oracle_pins.HAND_PLAN, (0, 1, 2, 3, 4, 5, 6), (249, 250, 251, 252, 253,
                                                                                              254, 255)])
def test_all_bit_patterns(zc, lib, plan):
    x = oracle_pins.all_patterns(seed=sum(plan))
    (y,), st = decode(zc, lib, [oracle.encode(x, plan)], [x.size])
    assert st[0] == 0 and np.array_equal(y, x)


def test_zero_point_densities_in_one_batch(zc, lib):
    n = 40_000
    Es = [0, 1, 100, 4096, 8192, 20_000, 39_999, 40_000]
    xs = [oracle_pins.with_escapes(n, E, 31 + E) for E in Es]
    ys, st = decode(zc, lib, [oracle.encode(x, WINDOW_PLAN) for x in xs], [n] * len(Es))
    assert not st.any()
    for y, x, E in zip(ys, xs, Es):
        assert np.array_equal(y, x), E


def test_batch_of_many_segments_with_raw_streams(zc, lib):
    """Many segments in one launch (block ranges of one or two tiles), empty and
    one-value ones, and raw streams: long ones, whose exact size reaches the
    coded layout (the coded decoder's raw branch), and short ones, whose exact
    size does not (the raw-only decoder)."""
    g = np.random.default_rng(5)
    coded_ns = [int(v) for v in g.integers(0, 70_000, 36)] + [0, 1, 8192, 8193]
    raw_ns = [5, 100, 30_000, 65_537]
    xs, ss, ns = [], [], []
    for i, n in enumerate(coded_ns):
        xs.append(gaussian(n, 0.01 * (1 + i % 5), 200 + i))
        ss.append(oracle.encode(xs[-1], WINDOW_PLAN))
        ns.append(n)
    for i, n in enumerate(raw_ns):
        x = oracle_pins.with_escapes(n, n, 100 + i)  # expands when coded: stored raw
        s = oracle.encode(x, WINDOW_PLAN, raw_fallback=True)
        assert s[31] == 1
        xs.append(x)
        ss.append(s)
        ns.append(n)
    short = [s.size < oracle.layout(n)["off_zp"] for s, n in zip(ss, ns)]
    assert any(short) and not all(short[len(coded_ns):])
    ys, st = decode(zc, lib, ss, ns)
    assert not st.any()
    for i, (y, x) in enumerate(zip(ys, xs)):
        assert np.array_equal(y, x), i


def test_bad_header_writes_nothing(zc, lib):
    n = 30_000
    x = gaussian(n, 0.02, 5)
    s = oracle.encode(x, WINDOW_PLAN)
    for pos in (0, 4, 8, 16, 20, 25, 31, 32, 40, 64, 127):
        bad = s.copy()
        bad[pos] ^= 0x40
        (y,), st = decode(zc, lib, [bad], [n])
        assert st[0] == zc.ZC_ERR_CORRUPT, pos
        assert (y == FILL).all(), pos


def test_table_and_plane_corruption_is_flagged(zc, lib):
    n = 50_000
    x = gaussian(n, 0.05, 6)
    s = oracle.encode(x, WINDOW_PLAN)
    lay = oracle.layout(n)
    zp_index = int(np.flatnonzero(~np.isin(oracle_pins.exponent_field(x), WINDOW_PLAN))[10])
    plane_pos = lay["off_p0"] + zp_index // 8
    for pos, bit in ((lay["off_tab"] + 4, 0x01), (lay["off_tab"] + 12, 0x01), (lay["off_tab"] + 8, 0x02),
                     (plane_pos, 1 << (zp_index % 8))):
        bad = s.copy()
        bad[pos] ^= bit
        _, st = decode(zc, lib, [bad], [n])
        assert st[0] == zc.ZC_ERR_CORRUPT, pos
