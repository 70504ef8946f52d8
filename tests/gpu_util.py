"""Device-side helpers for the GPU tests: torch provides memory and the stream,
the C ABI (through the ctypes binding) does all codec work."""
from __future__ import annotations

import numpy as np
import torch

SLOT_ALIGN = 256


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device; none is visible")
    from lossless_bf16_exponent_amd import zc  # raises if libzc.so is missing
    return zc


def to_device(x: np.ndarray) -> torch.Tensor:
    """uint16 BF16 patterns -> int16 device tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).cuda()


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def slot(nbytes: int) -> int:
    return (nbytes + SLOT_ALIGN - 1) // SLOT_ALIGN * SLOT_ALIGN


class Encoded:
    def __init__(self, buf, offsets, totals, caps):
        self.buf, self.offsets, self.totals, self.caps = buf, offsets, totals, caps

    def stream(self, i: int) -> np.ndarray:
        o = self.offsets[i]
        return self.buf[o:o + int(self.totals[i])].cpu().numpy()


def compress_batch(zc, xs_dev, ns, plans, batch: bool = True, fill: int = 0xA5) -> Encoded:
    """Compress segments (device tensors or views) into one buffer with one slot
    per segment; batch=False issues one zc_compress per segment instead."""
    caps = [zc.zc_max_compressed_bytes(n) for n in ns]
    offsets, off = [], 0
    for c in caps:
        offsets.append(off)
        off += slot(c)
    buf = torch.full((max(off, SLOT_ALIGN),), fill, dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(len(ns), dtype=torch.int64, device="cuda")
    base = buf.data_ptr()
    segs = [(x, n, p, base + o, c, sizes.data_ptr() + 8 * i)
            for i, (x, n, p, o, c) in enumerate(zip(xs_dev, ns, plans, offsets, caps))]
    if batch:
        zc.zc_compress_batch(segs)
    else:
        for s in segs:
            zc.zc_compress(*s)
    torch.cuda.synchronize()
    return Encoded(buf, offsets, sizes.cpu().numpy(), caps)


def decompress_batch(zc, enc: Encoded, ns, batch: bool = True, fill: int = 0x5A5A, in_bytes=None):
    outs = [torch.full((max(n, 1),), fill - 65536 if fill > 32767 else fill, dtype=torch.int16, device="cuda")
            for n in ns]
    status = torch.full((len(ns),), -1, dtype=torch.int32, device="cuda")
    base = enc.buf.data_ptr()
    segs = []
    for i, n in enumerate(ns):
        nb = int(enc.totals[i]) if in_bytes is None else in_bytes[i]
        segs.append((base + enc.offsets[i], nb, n, outs[i], status.data_ptr() + 4 * i))
    if batch:
        zc.zc_decompress_batch(segs)
    else:
        for s in segs:
            zc.zc_decompress(*s)
    torch.cuda.synchronize()
    return outs, status.cpu().numpy()
