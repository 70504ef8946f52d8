"""The histogram entry point that allocates nothing (its workspace is the
library's static device array) against zc_exponent_histogram with a caller
workspace: equal counts, exactly, on calls in a row (the second smaller, so a
stale row of the first call would show), with ragged sizes and the
special-value patterns."""
import numpy as np
import pytest
import torch

from gpu_util import require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zc():
    return require_gpu()


def histograms(zc, x_dev, n):
    ws = torch.empty(zc.zc_stats_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    ref = torch.full((256,), -1, dtype=torch.int64, device="cuda")
    got = torch.full((256,), -1, dtype=torch.int64, device="cuda")
    zc.zc_exponent_histogram(x_dev, n, ws, ws.numel(), ref)
    zc.zc_exponent_histogram_noalloc(x_dev, n, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def gaussian(n, sigma, seed):
    from lossless_bf16_exponent_amd import workloads
    g = np.random.default_rng(seed)
    return workloads.bf16_bits_from_f32((g.standard_normal(n) * sigma).astype(np.float32))


@pytest.mark.parametrize("sizes", [(5_000_003, 300_001), (1 << 24, 4097), (65_536 * 3, 0)])
def test_noalloc_histogram_equals_workspace_histogram(zc, sizes):
    for i, n in enumerate(sizes):
        x = gaussian(n, (0.02, 3e-4)[i], 11 * n + i)
        if n >= 65_536:
            x[:65_536] = np.arange(65_536, dtype=np.uint16)  # every exponent field, NaN and Inf included
        x_dev = to_device(x) if n else torch.empty(8, dtype=torch.int16, device="cuda")
        ref, got = histograms(zc, x_dev, n)
        assert int(ref.sum()) == n
        assert np.array_equal(got, ref), (n, np.flatnonzero(got != ref)[:8])


def test_noalloc_histogram_stream_ordered_with_other_work(zc):
    """Two inputs on one stream, back to back with no synchronization between
    them: each result equals its own workspace histogram."""
    a = to_device(gaussian(2_000_001, 1.0, 1))
    b = to_device(gaussian(777_777, 1e-3, 2))
    ha = torch.empty(256, dtype=torch.int64, device="cuda")
    hb = torch.empty(256, dtype=torch.int64, device="cuda")
    zc.zc_exponent_histogram_noalloc(a, a.numel(), ha)
    zc.zc_exponent_histogram_noalloc(b, b.numel(), hb)
    torch.cuda.synchronize()
    for x, h in ((a, ha), (b, hb)):
        ref, _ = histograms(zc, x, x.numel())
        assert np.array_equal(h.cpu().numpy(), ref)


def test_noalloc_histogram_rejects_bad_arguments(zc):
    x = torch.zeros(64, dtype=torch.int16, device="cuda")
    h = torch.zeros(256, dtype=torch.int64, device="cuda")
    with pytest.raises(zc.ZcError) as e:
        zc.zc_exponent_histogram_noalloc(x, 64, None)
    assert e.value.status == zc.ZC_ERR_INVALID_ARG
    with pytest.raises(zc.ZcError) as e:
        zc.zc_exponent_histogram_noalloc(x.data_ptr() + 2, 8, h)
    assert e.value.status == zc.ZC_ERR_MISALIGNED
    with pytest.raises(zc.ZcError) as e:
        zc.zc_exponent_histogram_noalloc(x, 1 << 32, h)
    assert e.value.status == zc.ZC_ERR_INVALID_ARG
