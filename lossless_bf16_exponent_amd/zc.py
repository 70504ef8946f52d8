"""Python binding of the C ABI in include/zc.h (argument marshalling only).

Every function has the name of the C entry point it calls.  Pointer arguments
accept an integer device address or anything with ``data_ptr()`` (a torch
tensor); ``stream`` accepts a raw hipStream_t integer, a ``torch.cuda.Stream``
or None for torch's current stream.  All compression work runs in the HIP
kernels of libzc.so; nothing here touches the data.

Importing this module fails loudly when libzc.so has not been built: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libzc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libzc.so is not built (run __graft_entry__.build() or "
                      "python -m lossless_bf16_exponent_amd._build); the codec has no fallback")

_lib = ctypes.CDLL(LIB_PATH)

ZC_OK, ZC_ERR_INVALID_ARG, ZC_ERR_CAPACITY, ZC_ERR_MISALIGNED, ZC_ERR_CORRUPT, ZC_ERR_HIP = range(6)
ZC_MAX_BATCH = 64
ZC_PLAN_RAW_FALLBACK = 1


class zc_plan(ctypes.Structure):
    _fields_ = [("exps", ctypes.c_uint8 * 7), ("flags", ctypes.c_uint8)]


class zc_enc_seg(ctypes.Structure):
    _fields_ = [("in_", ctypes.c_void_p), ("n", ctypes.c_uint64), ("plan", zc_plan),
                ("out", ctypes.c_void_p), ("out_capacity", ctypes.c_uint64), ("out_bytes", ctypes.c_void_p)]


class zc_dec_seg(ctypes.Structure):
    _fields_ = [("in_", ctypes.c_void_p), ("in_bytes", ctypes.c_uint64), ("n", ctypes.c_uint64),
                ("out", ctypes.c_void_p), ("status", ctypes.c_void_p)]


class zc_stream_info(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint64), ("zero_points", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64),
                ("groups", ctypes.c_uint32), ("plan", zc_plan), ("raw", ctypes.c_uint32)]


_lib.zc_plan_from_sigma.argtypes = [ctypes.c_double, ctypes.POINTER(zc_plan)]
_lib.zc_plan_from_sigma.restype = ctypes.c_int
_lib.zc_max_compressed_bytes.argtypes = [ctypes.c_uint64]
_lib.zc_max_compressed_bytes.restype = ctypes.c_uint64
_lib.zc_compress.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(zc_plan), ctypes.c_void_p,
                             ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
_lib.zc_compress.restype = ctypes.c_int
_lib.zc_compress_workspace_bytes.argtypes = [ctypes.c_uint64]
_lib.zc_compress_workspace_bytes.restype = ctypes.c_uint64
_lib.zc_compress_ws.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(zc_plan), ctypes.c_void_p,
                                ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
_lib.zc_compress_ws.restype = ctypes.c_int
_lib.zc_compress_batch_ws.argtypes = [ctypes.POINTER(zc_enc_seg), ctypes.c_uint32, ctypes.c_void_p, ctypes.c_uint64,
                                      ctypes.c_void_p]
_lib.zc_compress_batch_ws.restype = ctypes.c_int
_lib.zc_decompress.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p]
_lib.zc_decompress.restype = ctypes.c_int
_lib.zc_compress_batch.argtypes = [ctypes.POINTER(zc_enc_seg), ctypes.c_uint32, ctypes.c_void_p]
_lib.zc_compress_batch.restype = ctypes.c_int
_lib.zc_decompress_batch.argtypes = [ctypes.POINTER(zc_dec_seg), ctypes.c_uint32, ctypes.c_void_p]
_lib.zc_decompress_batch.restype = ctypes.c_int
_lib.zc_decompress_reduce.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_uint64),
                                     ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
_lib.zc_decompress_reduce.restype = ctypes.c_int
_lib.zc_stats_workspace_bytes.argtypes = [ctypes.c_uint64]
_lib.zc_stats_workspace_bytes.restype = ctypes.c_uint64
_lib.zc_exponent_histogram.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64,
                                       ctypes.c_void_p, ctypes.c_void_p]
_lib.zc_exponent_histogram.restype = ctypes.c_int
_lib.zc_exponent_histogram_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
_lib.zc_exponent_histogram_noalloc.restype = ctypes.c_int
_lib.zc_plan_from_histogram.argtypes = [ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(zc_plan)]
_lib.zc_plan_from_histogram.restype = ctypes.c_int
_lib.zc_estimate_sigma.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.zc_estimate_sigma.restype = ctypes.c_int
_lib.zc_read_header.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(zc_stream_info)]
_lib.zc_read_header.restype = ctypes.c_int
_lib.zc_status_string.argtypes = [ctypes.c_int]
_lib.zc_status_string.restype = ctypes.c_char_p

EXPORTED = ("zc_plan_from_sigma", "zc_max_compressed_bytes", "zc_compress", "zc_decompress",
            "zc_compress_batch", "zc_decompress_batch", "zc_decompress_reduce", "zc_read_header",
            "zc_status_string", "zc_stats_workspace_bytes", "zc_exponent_histogram", "zc_plan_from_histogram",
            "zc_estimate_sigma", "zc_exponent_histogram_noalloc", "zc_compress_workspace_bytes", "zc_compress_ws",
            "zc_compress_batch_ws")


class ZcError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (status %d)" % (where, zc_status_string(status), status))
        self.status = status


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> int:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _plan(exps) -> zc_plan:
    if isinstance(exps, zc_plan):
        return exps
    exps = tuple(int(e) for e in exps)
    if len(exps) != 7:
        raise ValueError("a plan has exactly seven exponents")
    return zc_plan((ctypes.c_uint8 * 7)(*exps), 0)


def plan_with_raw_fallback(exps) -> zc_plan:
    """The plan `exps` with ZC_PLAN_RAW_FALLBACK set (pass it wherever a plan goes)."""
    p = _plan(tuple(exps.exps) if isinstance(exps, zc_plan) else exps)
    return zc_plan(p.exps, ZC_PLAN_RAW_FALLBACK)


def _check(rc: int, where: str) -> None:
    if rc != ZC_OK:
        raise ZcError(rc, where)


def zc_status_string(status: int) -> str:
    return _lib.zc_status_string(int(status)).decode()


def zc_plan_from_sigma(sigma: float) -> tuple:
    p = zc_plan()
    _check(_lib.zc_plan_from_sigma(float(sigma), ctypes.byref(p)), "zc_plan_from_sigma")
    return tuple(int(v) for v in p.exps)


def zc_max_compressed_bytes(n: int) -> int:
    return int(_lib.zc_max_compressed_bytes(int(n)))


def zc_compress_workspace_bytes(n: int) -> int:
    return int(_lib.zc_compress_workspace_bytes(int(n)))


def zc_compress_capacity(n: int) -> int:
    """Output capacity zc_compress / zc_compress_batch need for n values (the
    stream bound and the encoder's scratch behind it)."""
    return zc_max_compressed_bytes(n) + zc_compress_workspace_bytes(n)


def zc_compress_ws(d_in, n, plan, d_out, out_capacity, d_out_bytes, d_workspace, workspace_bytes,
                   stream=None) -> None:
    p = _plan(plan)
    _check(_lib.zc_compress_ws(_ptr(d_in), int(n), ctypes.byref(p), _ptr(d_out), int(out_capacity),
                               _ptr(d_out_bytes), _ptr(d_workspace), int(workspace_bytes), _stream(stream)),
           "zc_compress_ws")


def zc_compress(d_in, n, plan, d_out, out_capacity, d_out_bytes=None, stream=None) -> None:
    p = _plan(plan)
    _check(_lib.zc_compress(_ptr(d_in), int(n), ctypes.byref(p), _ptr(d_out), int(out_capacity),
                            _ptr(d_out_bytes), _stream(stream)), "zc_compress")


def zc_decompress(d_in, in_bytes, n, d_out, d_status=None, stream=None) -> None:
    _check(_lib.zc_decompress(_ptr(d_in), int(in_bytes), int(n), _ptr(d_out), _ptr(d_status),
                              _stream(stream)), "zc_decompress")


def zc_decompress_reduce(d_streams, in_bytes, n, d_local, d_out, d_status=None, stream=None) -> None:
    """d_streams / in_bytes: sequences of k stream pointers and their readable sizes."""
    d_streams, in_bytes = list(d_streams), list(in_bytes)
    k = len(d_streams)
    ptrs = (ctypes.c_void_p * max(1, k))(*[_ptr(p) for p in d_streams])
    sizes = (ctypes.c_uint64 * max(1, k))(*[int(b) for b in in_bytes])
    _check(_lib.zc_decompress_reduce(ptrs, sizes, k, int(n), _ptr(d_local), _ptr(d_out), _ptr(d_status),
                                     _stream(stream)), "zc_decompress_reduce")


def zc_stats_workspace_bytes(n: int) -> int:
    return int(_lib.zc_stats_workspace_bytes(int(n)))


def zc_exponent_histogram(d_in, n, d_workspace, workspace_bytes, d_hist, stream=None) -> None:
    _check(_lib.zc_exponent_histogram(_ptr(d_in), int(n), _ptr(d_workspace), int(workspace_bytes), _ptr(d_hist),
                                      _stream(stream)), "zc_exponent_histogram")


def zc_exponent_histogram_noalloc(d_in, n, d_hist, stream=None) -> None:
    _check(_lib.zc_exponent_histogram_noalloc(_ptr(d_in), int(n), _ptr(d_hist), _stream(stream)),
           "zc_exponent_histogram_noalloc")


def zc_plan_from_histogram(hist) -> tuple:
    """hist: 256 counts (any sequence of non-negative integers) held on the host."""
    counts = [int(v) for v in hist]
    if len(counts) != 256:
        raise ValueError("a histogram has 256 counts")
    h = (ctypes.c_uint64 * 256)(*counts)
    p = zc_plan()
    _check(_lib.zc_plan_from_histogram(h, ctypes.byref(p)), "zc_plan_from_histogram")
    return tuple(int(v) for v in p.exps)


def zc_estimate_sigma(d_in, n, d_workspace, workspace_bytes, d_sigma, d_finite=None, stream=None) -> None:
    _check(_lib.zc_estimate_sigma(_ptr(d_in), int(n), _ptr(d_workspace), int(workspace_bytes), _ptr(d_sigma),
                                  _ptr(d_finite), _stream(stream)), "zc_estimate_sigma")


def make_enc_segs(segs) -> ctypes.Array:
    """segs: iterable of (in, n, plan, out, out_capacity, out_bytes) tuples."""
    segs = list(segs)
    arr = (zc_enc_seg * max(1, len(segs)))()
    for i, (d_in, n, plan, d_out, cap, d_bytes) in enumerate(segs):
        arr[i] = zc_enc_seg(_ptr(d_in), int(n), _plan(plan), _ptr(d_out), int(cap), _ptr(d_bytes))
    return arr, len(segs)


def make_dec_segs(segs) -> ctypes.Array:
    """segs: iterable of (in, in_bytes, n, out, status) tuples."""
    segs = list(segs)
    arr = (zc_dec_seg * max(1, len(segs)))()
    for i, (d_in, in_bytes, n, d_out, d_status) in enumerate(segs):
        arr[i] = zc_dec_seg(_ptr(d_in), int(in_bytes), int(n), _ptr(d_out), _ptr(d_status))
    return arr, len(segs)


def zc_compress_batch(segs, stream=None) -> None:
    """segs: a (ctypes array, count) pair from make_enc_segs, or tuples for it."""
    arr, k = segs if isinstance(segs, tuple) and len(segs) == 2 and isinstance(segs[0], ctypes.Array) \
        else make_enc_segs(segs)
    _check(_lib.zc_compress_batch(arr, k, _stream(stream)), "zc_compress_batch")


def zc_compress_batch_ws(segs, d_workspace, workspace_bytes, stream=None) -> None:
    """zc_compress_batch with every segment's scratch in one workspace."""
    arr, k = segs if isinstance(segs, tuple) and len(segs) == 2 and isinstance(segs[0], ctypes.Array) \
        else make_enc_segs(segs)
    _check(_lib.zc_compress_batch_ws(arr, k, _ptr(d_workspace), int(workspace_bytes), _stream(stream)),
           "zc_compress_batch_ws")


def zc_decompress_batch(segs, stream=None) -> None:
    arr, k = segs if isinstance(segs, tuple) and len(segs) == 2 and isinstance(segs[0], ctypes.Array) \
        else make_dec_segs(segs)
    _check(_lib.zc_decompress_batch(arr, k, _stream(stream)), "zc_decompress_batch")


def zc_read_header(header: bytes) -> dict:
    buf = ctypes.create_string_buffer(bytes(header), len(header))
    info = zc_stream_info()
    _check(_lib.zc_read_header(buf, len(header), ctypes.byref(info)), "zc_read_header")
    return {"n": int(info.n), "zero_points": int(info.zero_points), "total_bytes": int(info.total_bytes),
            "groups": int(info.groups), "plan": tuple(int(v) for v in info.plan.exps), "raw": bool(info.raw)}


def raw_status(fn: str, *args) -> int:
    """Call a C entry point and return its status code without raising (for tests
    of the host-side argument checks)."""
    return int(getattr(_lib, fn)(*args))
