"""Compress and decompress captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed with new inputs: after every replay each stream equals the oracle's
for that replay's input, byte for byte, and decodes back to it.

The blocks of a compress launch hand counts and offsets to each other through
words in the segment's scratch, each word marked with the launch's token, so
that words left by earlier calls never pass for current ones.  A replay runs
with the arguments that were captured; the token must still change from one
replay to the next.  Cases: a staged batch (more spans than the device holds
at once), a direct launch, and segments under the raw fallback whose outcome
flips between coded and raw from one replay to the next (two launches per
call); the scratch in a workspace or behind each stream; an eager call on the
same buffers between two replays.  The other entry points (the local
reduction, the histograms, the sigma estimate) pass no words between
workgroups; one case replays them too."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import require_gpu, slot, to_host_u16
from lossless_bf16_exponent_amd import workloads

pytestmark = pytest.mark.gpu

SPAN = 8192


@pytest.fixture(scope="module")
def zc():
    return require_gpu()


def gaussian(g, n: int, sigma: float) -> np.ndarray:
    return workloads.bf16_bits_from_f32(g.standard_normal(n).astype(np.float32) * np.float32(sigma))


def uniform_patterns(g, n: int) -> np.ndarray:
    """Any BF16 pattern but NaN/Inf: coding expands these (raw under the fallback)."""
    x = g.integers(0, 1 << 16, n).astype(np.uint16)
    return np.where((x & 0x7F80) == 0x7F80, x & 0x807F, x).astype(np.uint16)


class Captured:
    """Buffers of one batch (inputs, outputs with their sizes, workspace,
    decode outputs) and a graph holding one compress and one decompress call."""

    def __init__(self, zc, ns, sigmas, flags, workspace: bool, tables=None):
        self.ns, self.sigmas, self.flags = ns, sigmas, flags
        plans = tables if tables is not None else [zc.zc_plan_from_sigma(s) for s in sigmas]
        self.exps = [tuple(p) for p in plans]
        plans = [zc.plan_with_raw_fallback(p) if f else p for p, f in zip(plans, flags)]
        self.caps = [zc.zc_max_compressed_bytes(n) if workspace else zc.zc_compress_capacity(n) for n in ns]
        offs = np.concatenate([[0], np.cumsum([slot(c) for c in self.caps])]).astype(np.int64)
        self.offs = offs
        self.x = [torch.zeros(max(n, 1), dtype=torch.int16, device="cuda") for n in ns]
        self.out = torch.zeros(int(offs[-1]), dtype=torch.uint8, device="cuda")
        self.sizes = torch.zeros(len(ns), dtype=torch.int64, device="cuda")
        self.dec = [torch.zeros(max(n, 1), dtype=torch.int16, device="cuda") for n in ns]
        self.status = torch.zeros(len(ns), dtype=torch.int32, device="cuda")
        ob = self.out.data_ptr()
        self.enc = zc.make_enc_segs([(self.x[i], n, plans[i], ob + int(offs[i]), self.caps[i],
                                      self.sizes.data_ptr() + 8 * i) for i, n in enumerate(ns)])
        self.decs = zc.make_dec_segs([(ob + int(offs[i]), self.caps[i], n, self.dec[i],
                                       self.status.data_ptr() + 4 * i) for i, n in enumerate(ns)])
        wsb = sum(zc.zc_compress_workspace_bytes(n) for n in ns)
        self.ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda") if workspace else None
        self.zc = zc

    def compress(self):
        if self.ws is not None:
            self.zc.zc_compress_batch_ws(self.enc, self.ws, self.ws.numel())
        else:
            self.zc.zc_compress_batch(self.enc)

    def both(self):
        self.compress()
        self.zc.zc_decompress_batch(self.decs)

    def capture(self) -> torch.cuda.CUDAGraph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.both()  # eager once before the capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.both()
        torch.cuda.synchronize()
        return graph

    def load(self, xs):
        for t, x in zip(self.x, xs):
            if x.size:
                t[:x.size].copy_(torch.from_numpy(x.view(np.int16)))
        for i, n in enumerate(self.ns):  # the stream areas only: scratch behind them keeps its words
            o = int(self.offs[i])
            self.out[o:o + self.zc.zc_max_compressed_bytes(n)].fill_(0xA5)
        self.status.fill_(-1)
        for d in self.dec:
            d.fill_(0x1357)
        torch.cuda.synchronize()

    def check(self, xs, what: str):
        sizes = self.sizes.cpu().numpy()
        assert not self.status.cpu().numpy().any(), what
        for i, (x, e, f) in enumerate(zip(xs, self.exps, self.flags)):
            ref = oracle.encode(x, e, raw_fallback=f)
            o = int(self.offs[i])
            got = self.out[o:o + int(sizes[i])].cpu().numpy()
            assert got.size == ref.size and np.array_equal(got, ref), (what, i, int(sizes[i]), ref.size)
            assert np.array_equal(to_host_u16(self.dec[i][:x.size]), x), (what, i)


def replays(zc, ns, sigmas, flags, workspace, make, rounds=4, tables=None, seed=None):
    c = Captured(zc, ns, sigmas, flags, workspace, tables)
    g = np.random.default_rng(4242 + sum(ns) if seed is None else seed)
    c.load(make(g, 0))
    graph = c.capture()
    for r in range(rounds):
        xs = make(g, r + 1)
        c.load(xs)
        print("replay %d: n=%s workspace=%s" % (r, ns, workspace), flush=True)
        graph.replay()
        torch.cuda.synchronize()
        c.check(xs, "replay %d" % r)
        if r == 1:  # an eager call on the same buffers between two replays
            xs = make(g, 100)
            c.load(xs)
            c.both()
            torch.cuda.synchronize()
            c.check(xs, "eager call between replays")


@pytest.mark.parametrize("workspace", [True, False])
def test_graph_staged_batch(zc, workspace):
    """Three segments, 2,703 spans: a staged launch (finalize blocks)."""
    ns = [1100 * SPAN + 37, 900 * SPAN, 703 * SPAN - 5]
    sigmas = [0.02, 0.003, 0.0005]
    # every replay: new values, and sigmas off the plans' by a replay-dependent
    # factor, so that the zero-point counts (and every offset) change
    replays(zc, ns, sigmas, [False] * 3, workspace,
            lambda g, r: [gaussian(g, n, s * (1.0 + 0.6 * (r % 3))) for n, s in zip(ns, sigmas)])


@pytest.mark.parametrize("workspace", [True, False])
def test_graph_direct(zc, workspace):
    """Two segments, 600 spans: a direct launch."""
    ns = [300 * SPAN + 11, 300 * SPAN]
    sigmas = [0.01, 0.05]
    replays(zc, ns, sigmas, [False, False], workspace,
            lambda g, r: [gaussian(g, n, s * (1.0 + 0.5 * (r % 2))) for n, s in zip(ns, sigmas)])


@pytest.mark.parametrize("ns", [[200 * SPAN, 50 * SPAN + 3], [2100 * SPAN, 40 * SPAN]],
                         ids=["direct", "staged"])
def test_graph_raw_fallback(zc, ns):
    """A flagged segment whose outcome flips between coded and raw from one
    replay to the next (the second launch then copies the payload or codes
    it), next to an unflagged one."""
    sigmas = [0.02, 0.02]

    def make(g, r):
        first = uniform_patterns(g, ns[0]) if r % 2 else gaussian(g, ns[0], sigmas[0])
        return [first, gaussian(g, ns[1], sigmas[1])]
    replays(zc, ns, sigmas, [True, False], True, make)


@pytest.mark.parametrize("case", range(8))
def test_graph_random_batches(zc, case):
    """Seeded random batches: 1-5 segments with sizes at the tiling's edges or
    random (one case in two with a segment over 2,048 spans), random tables,
    the raw-fallback flag and the workspace drawn per case; every replay draws
    new values with a new zero-point share per segment."""
    from test_gpu_random import random_plan, random_size, random_values
    g = np.random.default_rng(5100 + case)
    k = int(g.integers(1, 6))
    ns = [random_size(g, case % 2 == 1 and i == 0) for i in range(k)]
    tables = [random_plan(g) for _ in range(k)]
    flags = [bool(g.random() < 0.35) for _ in range(k)]
    workspace = bool(g.random() < 0.5)
    print("graph random case %d: n=%s raw-fallback=%s workspace=%s" % (case, ns, flags, workspace), flush=True)

    def make(gr, r):
        return [random_values(gr, n, t, float(gr.choice([0.0, 0.01, 0.3, 1.0]))) for n, t in zip(ns, tables)]
    replays(zc, ns, [None] * k, flags, workspace, make, rounds=3, tables=tables, seed=6100 + case)


def test_graph_reduce_and_statistics(zc):
    """The local reduction of peer streams, the exponent histogram (with a
    workspace, and the no-allocation form) and the sigma estimate captured in
    one graph and replayed with new inputs; the peer streams are compressed
    eagerly before each replay.  The reduction and both histograms equal the
    oracle's; the sigma estimate equals that of an eager call on the same
    input, bit for bit (its grid is fixed)."""
    n, sigmas = 1_500_003, (0.01, 0.02, 0.005)
    k = len(sigmas)
    exps = [tuple(zc.zc_plan_from_sigma(s)) for s in sigmas]
    cap = zc.zc_max_compressed_bytes(n)
    streams = torch.zeros((k, slot(cap)), dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(k, dtype=torch.int64, device="cuda")
    enc_ws = torch.zeros(zc.zc_compress_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    peers = [torch.zeros(n, dtype=torch.int16, device="cuda") for _ in range(k)]
    local = torch.zeros(n, dtype=torch.int16, device="cuda")
    out = torch.zeros(n, dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(zc.zc_stats_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    hist = torch.zeros(256, dtype=torch.int64, device="cuda")
    hist_na = torch.zeros(256, dtype=torch.int64, device="cuda")
    sig = torch.zeros(2, dtype=torch.int64, device="cuda")  # sigma bits, finite count
    ptrs = [streams[i].data_ptr() for i in range(k)]

    def body():
        zc.zc_decompress_reduce(ptrs, [cap] * k, n, local, out, status)
        zc.zc_exponent_histogram(local, n, ws, ws.numel(), hist)
        zc.zc_exponent_histogram_noalloc(local, n, hist_na)
        zc.zc_estimate_sigma(local, n, ws, ws.numel(), sig.data_ptr(), sig.data_ptr() + 8)

    g = np.random.default_rng(77)

    def load(r):
        xs = [gaussian(g, n, s * (1.0 + 0.5 * (r % 3))) for s in sigmas]
        x_local = gaussian(g, n, 0.01 * (1 + r))
        for t, x in zip(peers, xs):
            t.copy_(torch.from_numpy(x.view(np.int16)))
        local.copy_(torch.from_numpy(x_local.view(np.int16)))
        for i in range(k):  # eager work between replays
            zc.zc_compress_ws(peers[i], n, exps[i], streams[i], cap, sizes.data_ptr() + 8 * i, enc_ws,
                              enc_ws.numel())
        out.fill_(0x1357)
        status.fill_(-1)
        torch.cuda.synchronize()
        return xs, x_local

    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    torch.cuda.synchronize()
    for r in range(4):
        xs, x_local = load(r + 1)
        print("replay %d: reduce of %d peers and statistics, n=%d" % (r, k, n), flush=True)
        graph.replay()
        torch.cuda.synchronize()
        refs = [oracle.encode(x, e) for x, e in zip(xs, exps)]
        sz = sizes.cpu().numpy()
        for i in range(k):
            assert np.array_equal(streams[i][:int(sz[i])].cpu().numpy(), refs[i]), (r, i)
        rc, want = oracle.decode_reduce(refs, n, x_local)
        assert rc == 0 and int(status.item()) == 0, r
        assert np.array_equal(to_host_u16(out), want), r
        h = oracle.exponent_histogram(x_local)
        assert np.array_equal(hist.cpu().numpy(), h) and np.array_equal(hist_na.cpu().numpy(), h), r
        got = sig.cpu().numpy().copy()
        sig.fill_(-1)
        zc.zc_estimate_sigma(local, n, ws, ws.numel(), sig.data_ptr(), sig.data_ptr() + 8)
        torch.cuda.synchronize()
        assert np.array_equal(got, sig.cpu().numpy()) and int(got[1]) == n, r
