"""The give-up path of compress.  Finalize work waits on words written by
other workgroups of the same launch; every wait is bounded, and a call whose
wait runs out must still end, leave a stream that every decoder rejects and
report a stream size of 0.  With workgroups dispatched in index order no wait
can run out, so the tests use builds of the library loaded next to the
shipped one: one whose spin limit is 0 (every wait gives up at once), and one
in which only the workgroups other than each segment's header writer act as
if a wait had run out (the header writer then learns of it only through the
segment's failure mark)."""
import ctypes
import os

import numpy as np
import pytest
import torch

from gpu_util import require_gpu, slot, to_device
from lossless_bf16_exponent_amd import _build, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zc():
    return require_gpu()


def load(zc, path):
    if not os.path.exists(path):
        raise RuntimeError("%s is not built (run __graft_entry__.build())" % path)
    lib = ctypes.CDLL(path)
    lib.zc_compress.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(zc.zc_plan), ctypes.c_void_p,
                                ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.zc_compress.restype = ctypes.c_int
    lib.zc_compress_batch.argtypes = [ctypes.POINTER(zc.zc_enc_seg), ctypes.c_uint32, ctypes.c_void_p]
    lib.zc_compress_batch.restype = ctypes.c_int
    return lib


@pytest.fixture(scope="module")
def giveup(zc):
    return load(zc, _build.GIVEUP_LIB)


@pytest.fixture(scope="module")
def failothers(zc):
    return load(zc, _build.FAIL_OTHERS_LIB)


def gaussian(n, sigma, seed):
    g = np.random.default_rng(seed)
    return workloads.bf16_bits_from_f32((g.standard_normal(n) * sigma).astype(np.float32))


def given_up_batch(zc, giveup, ns, sigmas, waits, raw_at=None):
    """Compress ns in one batched launch with a test build (giveup): segments
    that give up (waits[i]) report size 0 and a zero magic, and the shipped
    decoder rejects them without writing; the others equal the oracle's
    streams."""
    import oracle
    plans = [zc.zc_plan_from_sigma(s) for s in sigmas]
    if raw_at is not None:
        plans[raw_at] = zc.plan_with_raw_fallback(plans[raw_at])
    xs = [gaussian(n, s, i) for i, (n, s) in enumerate(zip(ns, sigmas))]
    devs = [to_device(x) if x.size else None for x in xs]
    caps = [zc.zc_compress_capacity(n) for n in ns]
    offs = np.concatenate([[0], np.cumsum([slot(c) for c in caps])]).astype(np.int64)
    buf = torch.full((int(offs[-1]),), 0x5A, dtype=torch.uint8, device="cuda")
    sizes = torch.full((len(ns),), 12345, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    arr, k = zc.make_enc_segs([(devs[i] if ns[i] else 0, ns[i], plans[i], buf.data_ptr() + int(offs[i]), caps[i],
                                sizes.data_ptr() + 8 * i) for i in range(len(ns))])
    assert giveup.zc_compress_batch(arr, k, stream.cuda_stream) == zc.ZC_OK
    torch.cuda.synchronize()  # the kernels ended
    got = sizes.cpu().numpy().tolist()
    for i in range(len(ns)):
        o = int(offs[i])
        magic = int.from_bytes(buf[o:o + 4].cpu().numpy().tobytes(), "little")
        if waits[i]:
            assert got[i] == 0 and magic == 0, i
        else:
            ref = oracle.encode(xs[i], plans[i])
            assert got[i] == ref.size and np.array_equal(buf[o:o + ref.size].cpu().numpy(), ref), i
    status = torch.full((len(ns),), -1, dtype=torch.int32, device="cuda")
    outs = [torch.full((max(n, 1),), 0x1357, dtype=torch.int16, device="cuda") for n in ns]
    zc.zc_decompress_batch([(buf.data_ptr() + int(offs[i]), caps[i], ns[i], outs[i], status.data_ptr() + 4 * i)
                            for i in range(len(ns))])
    torch.cuda.synchronize()
    assert status.cpu().numpy().tolist() == [zc.ZC_ERR_CORRUPT if w else 0 for w in waits]
    for o, w in zip(outs, waits):
        if w:
            assert bool((o == 0x1357).all())
    return xs, plans, devs, buf, caps, sizes


def test_given_up_staged_launch(zc, giveup):
    """A launch of more than 2048 spans is staged: every segment's finalize
    blocks wait for its encoder blocks, so every segment gives up (the
    one-span n = 0 segment too)."""
    ns = [300_007, 20_000_003, 8192 * 40 + 5, 1_000_003, 0]
    given_up_batch(zc, giveup, ns, (0.02, 1.0, 1e-3, 0.16, 1.0), [True] * len(ns), raw_at=3)


def test_given_up_direct_launch_and_single_call(zc, giveup):
    """A launch of at most 2048 spans is direct: a span waits for the spans
    before it, so a segment of more than one span gives up; a one-span segment
    waits for nothing and completes.  Then a single call, and the shipped
    library in the same process still compresses correctly."""
    import oracle
    ns = [300_007, 0, 8192 * 40 + 5, 1_000_003, 8000]
    xs, plans, devs, buf, caps, sizes = given_up_batch(zc, giveup, ns, (0.02, 1.0, 1e-3, 0.16, 0.5),
                                                      [n > 8192 for n in ns], raw_at=3)
    stream = torch.cuda.current_stream()
    sizes.fill_(12345)
    p0 = zc._plan(plans[0])
    rc = giveup.zc_compress(devs[0].data_ptr(), ns[0], ctypes.byref(p0), buf.data_ptr(), caps[0],
                            sizes.data_ptr(), stream.cuda_stream)
    assert rc == zc.ZC_OK
    torch.cuda.synchronize()
    assert int(sizes[0].item()) == 0
    assert int.from_bytes(buf[0:4].cpu().numpy().tobytes(), "little") == 0

    zc.zc_compress(devs[0], ns[0], plans[0], buf, caps[0], sizes)
    torch.cuda.synchronize()
    ref = oracle.encode(xs[0], plans[0])
    assert int(sizes[0].item()) == ref.size
    assert np.array_equal(buf[:ref.size].cpu().numpy(), ref)


def test_failure_mark_alone_invalidates(zc, failothers):
    """A build in which every finalize block and direct span other than a
    segment's header writer acts as if a wait had run out, while the header
    writer's own waits pass: the header writer finds only the failure mark,
    and must still leave an invalid stream.  A segment whose header writer is
    its only waiting block (one run of finalize work, or one direct span)
    completes and equals the oracle's stream."""
    # staged: 20,000,003 values are 2,442 spans (153 runs); 81,920 values 10 spans (one run)
    ns = [20_000_003, 8192 * 10, 300_007, 0]
    given_up_batch(zc, failothers, ns, (1.0, 0.02, 1e-3, 1.0), [True, False, True, False], raw_at=2)
    # direct: spans after the first wait for earlier ones; a one-span segment has no other block
    ns = [300_007, 0, 8000, 8192 * 40 + 5]
    given_up_batch(zc, failothers, ns, (0.02, 1.0, 0.5, 1e-3), [True, False, False, True])
