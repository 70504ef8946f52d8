"""CPU oracle of the BF16 exponent-coding codec -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does, and the two
share no code: the oracle is the plain C file ``zc_oracle.c`` next to this
module, built with gcc and loaded with ctypes.

The arithmetic follows the explainer pages of "ZipCCL: Efficient Lossless Data
Compression of Communication Collectives for Accelerating LLM Training"
(technical summary, sections 2.A and 2.B, the plan variants -- histogram and
sigma estimate -- that section 2.A contrasts with the closed form, and the
local reduction of the reduce-scatter path in section 2.D); the C file states
every step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "zc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_default = None
_lock = threading.Lock()

OK, ERR_INVALID_ARG, ERR_CAPACITY, ERR_CORRUPT = 0, 1, 2, 4


def compile_source(src_path: str, out_path: str) -> str:
    """gcc -O2 of one oracle source file into a shared library (no HIP, no GPU)."""
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, src_path, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    """Compile zc_oracle.c into liboracle.so next to it."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(SOURCE, _LIB_PATH)
    return _LIB_PATH


class Oracle:
    """ctypes view of one build of the oracle (the shipped one, or a test's mutant)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        lib.zco_exponent_probabilities.argtypes = [ctypes.c_double, ctypes.POINTER(ctypes.c_double)]
        lib.zco_exponent_probabilities.restype = ctypes.c_int
        lib.zco_plan_from_sigma.argtypes = [ctypes.c_double, u8p]
        lib.zco_plan_from_sigma.restype = ctypes.c_int
        lib.zco_layout.argtypes = [ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)]
        lib.zco_layout.restype = None
        lib.zco_max_bytes.argtypes = [ctypes.c_uint64]
        lib.zco_max_bytes.restype = ctypes.c_uint64
        lib.zco_encode.argtypes = [ctypes.c_void_p, ctypes.c_uint64, u8p, ctypes.c_void_p,
                                   ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)]
        lib.zco_encode.restype = ctypes.c_int
        lib.zco_encode_fallback.argtypes = lib.zco_encode.argtypes
        lib.zco_encode_fallback.restype = ctypes.c_int
        lib.zco_decode.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        lib.zco_decode.restype = ctypes.c_int
        lib.zco_decode_reduce.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_uint64),
                                          ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        lib.zco_decode_reduce.restype = ctypes.c_int
        lib.zco_float_to_bf16.argtypes = [ctypes.c_float]
        lib.zco_float_to_bf16.restype = ctypes.c_uint16
        lib.zco_exponent_histogram.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)]
        lib.zco_exponent_histogram.restype = None
        lib.zco_plan_from_histogram.argtypes = [ctypes.POINTER(ctypes.c_uint64), u8p]
        lib.zco_plan_from_histogram.restype = ctypes.c_int
        lib.zco_estimate_sigma.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)]
        lib.zco_estimate_sigma.restype = ctypes.c_double
        self.lib = lib
        self.path = path

    def exponent_probabilities(self, sigma: float) -> np.ndarray:
        """p[e] = P(a draw of N(0, sigma^2) has BF16 exponent field e), e = 0..255."""
        p = (ctypes.c_double * 256)()
        if self.lib.zco_exponent_probabilities(float(sigma), p) != OK:
            raise ValueError("invalid sigma %r" % (sigma,))
        return np.array(p[:], dtype=np.float64)

    def plan_from_sigma(self, sigma: float) -> tuple:
        """The seven most probable exponents under N(0, sigma^2), ascending."""
        buf = (ctypes.c_uint8 * 7)()
        if self.lib.zco_plan_from_sigma(float(sigma), buf) != OK:
            raise ValueError("invalid sigma %r" % (sigma,))
        return tuple(int(v) for v in buf)

    def layout(self, n: int) -> dict:
        out = (ctypes.c_uint64 * 7)()
        self.lib.zco_layout(int(n), out)
        keys = ("off_sm", "off_p0", "off_p1", "off_p2", "off_tab", "off_zp", "groups")
        return {k: int(v) for k, v in zip(keys, out)}

    def max_bytes(self, n: int) -> int:
        return int(self.lib.zco_max_bytes(int(n)))

    def encode(self, x: np.ndarray, exps, raw_fallback: bool = False) -> np.ndarray:
        """Compressed stream (uint8 array of exactly total_bytes) of BF16 patterns x;
        with raw_fallback, the raw stream whenever the coded one would be larger."""
        x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
        cap = self.max_bytes(x.size)
        out = np.empty(cap, dtype=np.uint8)
        total = self.encode_into(x, exps, out, raw_fallback)
        return out[:total]

    def encode_into(self, x: np.ndarray, exps, out: np.ndarray, raw_fallback: bool = False) -> int:
        """Encode into a caller buffer; returns total bytes."""
        total = ctypes.c_uint64(0)
        fn = self.lib.zco_encode_fallback if raw_fallback else self.lib.zco_encode
        rc = fn(x.ctypes.data, x.size, _plan_buf(exps), out.ctypes.data, out.size, ctypes.byref(total))
        if rc != OK:
            raise ValueError("oracle encode failed with status %d" % rc)
        return int(total.value)

    def decode(self, stream: np.ndarray, n: int):
        """(status, BF16 patterns).  status is 0 on success, 4 for a rejected stream."""
        stream = np.ascontiguousarray(stream, dtype=np.uint8).reshape(-1)
        out = np.zeros(int(n), dtype=np.uint16)
        return self.decode_into(stream, n, out), out

    def decode_into(self, stream: np.ndarray, n: int, out: np.ndarray) -> int:
        return int(self.lib.zco_decode(stream.ctypes.data, stream.size, int(n), out.ctypes.data))

    def decode_reduce(self, streams, n: int, local=None):
        """(status, BF16 patterns): the float32 sum of local (if given) and the
        decoded streams, in that order, rounded to BF16 (section 2.D reading)."""
        streams = [np.ascontiguousarray(s, dtype=np.uint8).reshape(-1) for s in streams]
        k = len(streams)
        ptrs = (ctypes.c_void_p * max(k, 1))(*[s.ctypes.data for s in streams])
        sizes = (ctypes.c_uint64 * max(k, 1))(*[s.size for s in streams])
        out = np.zeros(max(int(n), 1), dtype=np.uint16)
        loc = None
        if local is not None:
            loc = np.ascontiguousarray(local, dtype=np.uint16).reshape(-1)
            if loc.size != n:
                raise ValueError("local has %d values, expected %d" % (loc.size, n))
        rc = self.lib.zco_decode_reduce(ptrs, sizes, k, int(n), None if loc is None else loc.ctypes.data,
                                        out.ctypes.data)
        return int(rc), out[:int(n)]

    def exponent_histogram(self, x: np.ndarray) -> np.ndarray:
        """Count of every BF16 exponent field (0..255) among the patterns x."""
        x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
        h = (ctypes.c_uint64 * 256)()
        self.lib.zco_exponent_histogram(x.ctypes.data, x.size, h)
        return np.array(h[:], dtype=np.uint64)

    def plan_from_histogram(self, hist) -> tuple:
        """The seven most frequent exponent fields, ascending (ties to the smaller)."""
        h = (ctypes.c_uint64 * 256)(*[int(v) for v in hist])
        buf = (ctypes.c_uint8 * 7)()
        self.lib.zco_plan_from_histogram(h, buf)
        return tuple(int(v) for v in buf)

    def estimate_sigma(self, x: np.ndarray):
        """(sigma, finite count): root mean square of the finite BF16 values."""
        x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
        m = ctypes.c_uint64(0)
        return float(self.lib.zco_estimate_sigma(x.ctypes.data, x.size, ctypes.byref(m))), int(m.value)

    def float_to_bf16(self, f: float) -> int:
        """Nearest BF16 pattern to a float32 value (ties to even; NaN -> 0x7FC0)."""
        return int(self.lib.zco_float_to_bf16(float(f)))


def _plan_buf(exps):
    exps = tuple(int(e) for e in exps)
    if len(exps) != 7:
        raise ValueError("a plan has exactly seven exponents")
    return (ctypes.c_uint8 * 7)(*exps)


def default() -> Oracle:
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            _default = Oracle(_LIB_PATH)
    return _default


def exponent_probabilities(sigma):
    return default().exponent_probabilities(sigma)


def plan_from_sigma(sigma):
    return default().plan_from_sigma(sigma)


def layout(n):
    return default().layout(n)


def max_bytes(n):
    return default().max_bytes(n)


def encode(x, exps, raw_fallback=False):
    return default().encode(x, exps, raw_fallback)


def encode_into(x, exps, out, raw_fallback=False):
    return default().encode_into(x, exps, out, raw_fallback)


def decode(stream, n):
    return default().decode(stream, n)


def decode_into(stream, n, out):
    return default().decode_into(stream, n, out)


def decode_reduce(streams, n, local=None):
    return default().decode_reduce(streams, n, local)


def float_to_bf16(f):
    return default().float_to_bf16(f)


def exponent_histogram(x):
    return default().exponent_histogram(x)


def plan_from_histogram(hist):
    return default().plan_from_histogram(hist)


def estimate_sigma(x):
    return default().estimate_sigma(x)
