"""Device-side helpers for the GPU tests: torch provides memory and the stream,
the C ABI (through the ctypes binding) does all codec work."""
from __future__ import annotations

import numpy as np
import torch

SLOT_ALIGN = 256
GUARD = 4096  # bytes of sentinel before and after every device output of the helpers


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


def load_test_build(zc, path: str):
    """A test build of the library (ctypes handle), loaded next to the shipped one."""
    import ctypes
    import os
    if not os.path.exists(path):
        raise RuntimeError("%s is not built (run __graft_entry__.build())" % path)
    lib = ctypes.CDLL(path)
    lib.zc_compress.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(zc.zc_plan), ctypes.c_void_p,
                                ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.zc_compress.restype = ctypes.c_int
    lib.zc_compress_batch.argtypes = [ctypes.POINTER(zc.zc_enc_seg), ctypes.c_uint32, ctypes.c_void_p]
    lib.zc_compress_batch.restype = ctypes.c_int
    lib.zc_compress_batch_ws.argtypes = [ctypes.POINTER(zc.zc_enc_seg), ctypes.c_uint32, ctypes.c_void_p,
                                         ctypes.c_uint64, ctypes.c_void_p]
    lib.zc_compress_batch_ws.restype = ctypes.c_int
    lib.zc_decompress_batch.argtypes = [ctypes.POINTER(zc.zc_dec_seg), ctypes.c_uint32, ctypes.c_void_p]
    lib.zc_decompress_batch.restype = ctypes.c_int
    return lib


def check_untouched(t: torch.Tensor, fill: int, what: str) -> None:
    """A sentinel region still holds its fill value everywhere."""
    if t.numel() and not bool((t == fill).all()):
        bad = torch.nonzero(t != fill).flatten()[:4].cpu().numpy()
        raise AssertionError("%s: sentinel bytes overwritten (first at %s)" % (what, bad))


def compress_batch(zc, xs_dev, ns, plans, batch: bool = True, fill: int = 0xA5, lib=None,
                   workspace: bool = False) -> Encoded:
    """Compress segments (device tensors or views) into one buffer with one slot
    per segment; batch=False issues one zc_compress per segment instead; lib: a
    test build of the library (ctypes handle) to call in place of the shipped
    one (batched calls only); workspace: the _ws calls, with the encoder's
    scratch in a separate workspace (filled with random bytes first) and slots
    of zc_max_compressed_bytes(n) only.  Every slot has GUARD sentinel bytes
    before it and after its capacity, checked untouched after the call."""
    caps = [zc.zc_max_compressed_bytes(n) if workspace else zc.zc_compress_capacity(n) for n in ns]
    offsets, off = [], GUARD
    for c in caps:
        offsets.append(off)
        off += slot(c) + GUARD
    buf = torch.full((off,), fill, dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(len(ns), dtype=torch.int64, device="cuda")
    base = buf.data_ptr()
    segs = [(x, n, p, base + o, c, sizes.data_ptr() + 8 * i)
            for i, (x, n, p, o, c) in enumerate(zip(xs_dev, ns, plans, offsets, caps))]
    if workspace:
        wsb = [zc.zc_compress_workspace_bytes(n) for n in ns]
        ws = torch.randint(0, 256, (sum(wsb) if batch else max(wsb),), dtype=torch.uint8, device="cuda")
        if batch:
            arr, k = zc.make_enc_segs(segs)
            if lib is not None:
                rc = lib.zc_compress_batch_ws(arr, k, ws.data_ptr(), ws.numel(),
                                              torch.cuda.current_stream().cuda_stream)
                assert rc == zc.ZC_OK, rc
            else:
                zc.zc_compress_batch_ws((arr, k), ws, ws.numel())
        else:
            for s in segs:  # one workspace, reused call after call on the stream
                zc.zc_compress_ws(*s, ws, ws.numel())
    elif lib is not None:
        arr, k = zc.make_enc_segs(segs)
        rc = lib.zc_compress_batch(arr, k, torch.cuda.current_stream().cuda_stream)
        assert rc == zc.ZC_OK, rc
    elif batch:
        zc.zc_compress_batch(segs)
    else:
        for s in segs:
            zc.zc_compress(*s)
    torch.cuda.synchronize()
    prev = 0
    for i, (o, c) in enumerate(zip(offsets, caps)):
        check_untouched(buf[prev:o], fill, "before the output of segment %d" % i)
        prev = o + c
    check_untouched(buf[prev:], fill, "after the last output")
    return Encoded(buf, offsets, sizes.cpu().numpy(), caps)


def decompress_batch(zc, enc: Encoded, ns, batch: bool = True, fill: int = 0x5A5A, in_bytes=None):
    """Decompress every stream of enc into its own output (a view with GUARD
    sentinel bytes on both sides, checked untouched after the call)."""
    g = GUARD // 2
    v = fill - 65536 if fill > 32767 else fill
    bufs = [torch.full((max(n, 1) + 2 * g,), v, dtype=torch.int16, device="cuda") for n in ns]
    outs = [b[g:g + max(n, 1)] for b, n in zip(bufs, ns)]
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
    for i, (b, n) in enumerate(zip(bufs, ns)):
        check_untouched(b[:g], v, "before the output of segment %d" % i)
        check_untouched(b[g + n:], v, "after the %d values of segment %d" % (n, i))
    return outs, status.cpu().numpy()
