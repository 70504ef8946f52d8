"""The largest tensor the format describes: n = 2^32 - 1 BF16 values (the
header's table and counts are 32-bit).  Seeded N(0, 0.02^2) values drawn on
the device.  The stream is compared with the oracle's byte for byte, it decodes
back to the input, the local reduction of the stream with the input as the
local share gives exactly 2x, and the exponent histogram and sigma estimate
agree with the oracle's.  Minutes of host work; marked slow."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import require_gpu, to_host_u16

pytestmark = pytest.mark.gpu

N_MAX = (1 << 32) - 1
U = 2.0 ** -53


@pytest.fixture(scope="module")
def zc():
    return require_gpu()


def say(msg):
    print(msg, flush=True)


@pytest.mark.slow
@pytest.mark.timeout(1200)
def test_maximum_size_round_trip(zc):
    n = N_MAX
    say("max size: drawing %d values on the device" % n)
    g = torch.Generator(device="cuda")
    g.manual_seed(20260)
    x = torch.empty(n, dtype=torch.int16, device="cuda")
    chunk = 1 << 28
    for s in range(0, n, chunk):  # float32 draws rounded to BF16 (nearest, ties to even)
        m = min(chunk, n - s)
        x[s:s + m] = (torch.randn(m, generator=g, device="cuda") * 0.02).to(torch.bfloat16).view(torch.int16)
    plan = zc.zc_plan_from_sigma(0.02)
    cap = zc.zc_max_compressed_bytes(n)  # the stream bound: the scratch goes to a workspace
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    wsb = zc.zc_compress_workspace_bytes(n)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    say("max size: compress (output %d bytes, workspace %d bytes)" % (cap, wsb))
    zc.zc_compress_ws(x, n, plan, out, cap, size, ws, wsb)
    torch.cuda.synchronize()
    total = int(size.item())
    del ws

    say("max size: decompress")
    dec = torch.empty_like(x)
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    zc.zc_decompress(out, total, n, dec, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and torch.equal(dec, x)
    del dec

    say("max size: local reduction of the stream with the input itself")
    red = torch.empty_like(x)
    zc.zc_decompress_reduce([out.data_ptr()], [total], n, x, red, st)
    torch.cuda.synchronize()
    twice = (x.view(torch.bfloat16).float() * 2).to(torch.bfloat16).view(torch.int16)  # exact: no overflow at 0.02
    assert int(st.item()) == 0 and torch.equal(red, twice)
    del red, twice

    say("max size: histogram and sigma on the device")
    ws = torch.empty(zc.zc_stats_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    hist = torch.zeros(256, dtype=torch.int64, device="cuda")
    zc.zc_exponent_histogram(x, n, ws, ws.numel(), hist)
    sig = torch.zeros(2, dtype=torch.float64, device="cuda")
    zc.zc_estimate_sigma(x, n, ws, ws.numel(), sig.data_ptr(), sig.data_ptr() + 8)
    torch.cuda.synchronize()
    h = hist.cpu().numpy().astype(np.uint64)
    s_dev = float(sig[0].item())
    m_dev = int(sig[1:].view(torch.int64).item())

    say("max size: copies to the host")
    xh = to_host_u16(x)
    got = out[:total].cpu().numpy()
    del out, x, ws
    torch.cuda.empty_cache()

    say("max size: oracle histogram and sigma")
    assert np.array_equal(h, oracle.exponent_histogram(xh)) and int(h.sum()) == n
    s_orc, m_orc = oracle.estimate_sigma(xh)
    assert m_dev == m_orc == n and abs(s_dev - s_orc) <= 2 * (n + 1024) * U * s_orc

    say("max size: oracle encode (about a minute)")
    ref = oracle.encode(xh, plan)
    say("max size: comparing %d stream bytes" % total)
    assert ref.size == total and np.array_equal(got, ref)
