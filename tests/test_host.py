"""Host-side checks of the HIP library that need no GPU: it loads and exports
every entry point of include/zc.h, its sigma plan equals the oracle's, every
host-detectable error returns its status before anything is enqueued, the
header parser agrees with oracle streams, the host histogram plan equals the
oracle's, and the per-lane bit helpers pass their CPU self-test."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle
import oracle_pins
from lossless_bf16_exponent_amd import _build, workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def zc():
    if not os.path.exists(_build.LIB):
        _build.build()
    from lossless_bf16_exponent_amd import zc as mod
    return mod


def declared_functions():
    text = open(os.path.join(ROOT, "include", "zc.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(zc_[a-z_]+)\s*\(", text, re.M)))


def test_exports_every_declared_entry_point(zc):
    names = declared_functions()
    assert len(names) >= 8
    out = subprocess.run(["nm", "-D", "--defined-only", _build.LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (zc_\w+)", out))
    for name in names:
        assert name in exported, name
        assert hasattr(zc._lib, name)
    assert set(zc.EXPORTED) == set(names)


def test_lane_helpers_selftest(tmp_path):
    exe = str(tmp_path / "lane_selftest")
    subprocess.run([_build.hipcc(), "-O2", "-std=c++17", "-x", "c++", "-I", _build.CSRC,
                    os.path.join(ROOT, "tests", "lane_selftest.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_compress_grid_layout_selftest(tmp_path):
    """Every span and finalize block gets one grid block, after all it waits for."""
    exe = str(tmp_path / "grid_selftest")
    subprocess.run([_build.hipcc(), "-O2", "-std=c++17", "-x", "c++", "-I", _build.CSRC,
                    os.path.join(ROOT, "tests", "grid_selftest.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


# ---------------------------------------------------------------------------
# the host-side C and C++ code under the address and undefined-behaviour
# sanitizers (host code only; no GPU code is built with them)
# ---------------------------------------------------------------------------

SANITIZE = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _clangxx() -> str:
    """The ROCm clang++ (its vector extensions build zc_lane.h on the host)."""
    cand = os.path.join(os.path.dirname(os.path.realpath(_build.hipcc())), "..", "llvm", "bin", "clang++")
    for c in (cand, "/opt/rocm/llvm/bin/clang++"):
        if os.path.exists(c):
            return c
    pytest.skip("the ROCm clang++ is not installed")


def _run_sanitized(cmd_build, exe):
    subprocess.run(cmd_build, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def test_host_abi_under_sanitizers(tmp_path):
    """zc_host.cpp (plans, capacity, header parser, status names) and the
    layout arithmetic, on edge and random inputs."""
    exe = str(tmp_path / "host_selftest")
    _run_sanitized(["g++", "-std=c++17", *SANITIZE, "-I", os.path.join(ROOT, "include"), "-I", _build.CSRC,
                    os.path.join(ROOT, "tests", "host_selftest.cpp"), os.path.join(_build.CSRC, "zc_host.cpp"),
                    "-o", exe], exe)


def test_grid_layout_under_sanitizers(tmp_path):
    exe = str(tmp_path / "grid_selftest_asan")
    _run_sanitized(["g++", "-std=c++17", *SANITIZE, "-I", _build.CSRC,
                    os.path.join(ROOT, "tests", "grid_selftest.cpp"), "-o", exe], exe)


def test_lane_helpers_under_sanitizers(tmp_path):
    exe = str(tmp_path / "lane_selftest_asan")
    _run_sanitized([_clangxx(), "-std=c++17", *SANITIZE, "-x", "c++", "-I", _build.CSRC,
                    os.path.join(ROOT, "tests", "lane_selftest.cpp"), "-o", exe], exe)


def test_oracle_pins_under_sanitizers(tmp_path):
    """Every oracle pin against a build of zc_oracle.c with the sanitizers, in a
    subprocess that preloads the address sanitizer's runtime."""
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", *SANITIZE, "-o", lib, oracle.SOURCE, "-lm"], check=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                             check=True).stdout.strip()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", LD_PRELOAD=libasan)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_sanitized.py"), lib],
                       capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert r.stdout.count("ok pin_") == len(oracle_pins.ALL_PINS)


def _near_tie(sigma):
    p = np.sort(oracle.exponent_probabilities(sigma))[::-1]
    return p[6] - p[7] < 1e-12


def test_library_plan_equals_oracle_plan(zc):
    sigmas = [0.02, 1.0, 0.16, 0.01, 1e-5, 1e38, 2.0 ** -130, 2.0 ** -120.7]
    sigmas += list(workloads.config3_sigmas())
    sigmas += [2.0 ** f for f in np.arange(-20.0, 20.0, 0.01)]
    checked = 0
    for s in sigmas:
        if _near_tie(s):
            continue
        assert zc.zc_plan_from_sigma(s) == oracle.plan_from_sigma(s), s
        checked += 1
    assert checked > 3900


def test_plan_rejects_bad_sigma(zc):
    for bad in (0.0, -0.5, float("nan"), float("inf"), -float("inf")):
        with pytest.raises(zc.ZcError) as e:
            zc.zc_plan_from_sigma(bad)
        assert e.value.status == zc.ZC_ERR_INVALID_ARG
    assert zc.raw_status("zc_plan_from_sigma", 0.02, None) == zc.ZC_ERR_INVALID_ARG


def test_max_compressed_bytes_covers_worst_stream(zc):
    """The stream bound covers the oracle's largest stream and the raw form and
    stays under 2.4 n for large n; the scratch is a little over n bytes."""
    for n in (0, 1, 63, 64, 4095, 4096, 4097, 8193, 1 << 20, 58_720_256, (1 << 30), (1 << 32) - 1):
        cap = zc.zc_max_compressed_bytes(n)
        ws = zc.zc_compress_workspace_bytes(n)
        assert cap >= oracle.max_bytes(n) and cap >= 128 + 2 * n, n
        assert cap % 128 == 0 and ws % 256 == 0 and ws >= n
        assert zc.zc_compress_capacity(n) == cap + ws
        if n >= 1 << 20:
            assert cap <= 2.4 * n and ws <= 1.01 * n + 16384, n
    assert zc.zc_max_compressed_bytes(1 << 32) == 0
    assert zc.zc_compress_workspace_bytes(1 << 32) == 0


FAKE_IN = 0x7F0000000000  # never dereferenced: every call below fails validation first
FAKE_OUT = 0x7F1000000000
PLAN = (116, 117, 118, 119, 120, 121, 122)


def _compress_status(zc, d_in=FAKE_IN, n=1000, plan=PLAN, flags=0, d_out=FAKE_OUT, cap=None, d_bytes=0):
    p = zc._plan(plan)
    p.flags = flags
    if cap is None:
        cap = zc.zc_compress_capacity(n) - 1  # one byte short: every other check must fire first
    return zc.raw_status("zc_compress", d_in, n, ctypes.byref(p), d_out, cap, d_bytes, 0)


def test_compress_host_errors(zc):
    assert _compress_status(zc) == zc.ZC_ERR_CAPACITY
    assert _compress_status(zc, d_out=0) == zc.ZC_ERR_INVALID_ARG
    assert _compress_status(zc, d_in=0) == zc.ZC_ERR_INVALID_ARG
    assert _compress_status(zc, n=1 << 32, cap=1 << 40) == zc.ZC_ERR_INVALID_ARG
    assert _compress_status(zc, plan=(116, 116, 118, 119, 120, 121, 122)) == zc.ZC_ERR_INVALID_ARG
    assert _compress_status(zc, plan=(122, 121, 120, 119, 118, 117, 116)) == zc.ZC_ERR_INVALID_ARG
    assert _compress_status(zc, flags=2) == zc.ZC_ERR_INVALID_ARG
    assert _compress_status(zc, flags=0x81) == zc.ZC_ERR_INVALID_ARG
    assert _compress_status(zc, flags=zc.ZC_PLAN_RAW_FALLBACK) == zc.ZC_ERR_CAPACITY  # a valid flag
    assert _compress_status(zc, d_in=FAKE_IN + 2) == zc.ZC_ERR_MISALIGNED
    assert _compress_status(zc, d_out=FAKE_OUT + 64) == zc.ZC_ERR_MISALIGNED
    assert _compress_status(zc, d_bytes=FAKE_OUT + 4) == zc.ZC_ERR_MISALIGNED
    assert zc.raw_status("zc_compress", FAKE_IN, 10, None, FAKE_OUT, 1 << 20, 0, 0) == zc.ZC_ERR_INVALID_ARG


def test_batch_host_errors(zc):
    arr, _ = zc.make_enc_segs([(FAKE_IN, 10, PLAN, FAKE_OUT, 1, 0)])
    assert zc.raw_status("zc_compress_batch", arr, 0, 0) == zc.ZC_ERR_INVALID_ARG
    assert zc.raw_status("zc_compress_batch", None, 1, 0) == zc.ZC_ERR_INVALID_ARG
    big, _ = zc.make_enc_segs([(FAKE_IN, 10, PLAN, FAKE_OUT, 1, 0)] * 65)
    assert zc.raw_status("zc_compress_batch", big, 65, 0) == zc.ZC_ERR_INVALID_ARG
    # one bad segment among good ones rejects the whole batch before any launch
    cap = zc.zc_compress_capacity(10)
    arr, k = zc.make_enc_segs([(FAKE_IN, 10, PLAN, FAKE_OUT, cap, 0),
                               (FAKE_IN, 10, PLAN, FAKE_OUT + (1 << 20), cap - 8, 0)])
    assert zc.raw_status("zc_compress_batch", arr, k, 0) == zc.ZC_ERR_CAPACITY
    darr, _ = zc.make_dec_segs([(FAKE_OUT, 1 << 20, 10, FAKE_IN, 0)])
    assert zc.raw_status("zc_decompress_batch", darr, 0, 0) == zc.ZC_ERR_INVALID_ARG
    dbig, _ = zc.make_dec_segs([(FAKE_OUT, 1 << 20, 10, FAKE_IN, 0)] * 65)
    assert zc.raw_status("zc_decompress_batch", dbig, 65, 0) == zc.ZC_ERR_INVALID_ARG


def test_workspace_host_errors(zc):
    """The _ws calls: a null or misaligned workspace, one too small (by a byte,
    or for a batch, short of the sum over its segments), and an output buffer
    short of the stream bound are rejected before any launch; the stream bound
    alone is enough output capacity."""
    n = 1000
    cap = zc.zc_max_compressed_bytes(n)
    wsb = zc.zc_compress_workspace_bytes(n)
    p = zc._plan(PLAN)
    WS = 0x7F2000000000
    st = lambda *a: zc.raw_status("zc_compress_ws", *a)
    assert st(FAKE_IN, n, ctypes.byref(p), FAKE_OUT, cap, 0, 0, wsb, 0) == zc.ZC_ERR_INVALID_ARG
    assert st(FAKE_IN, n, ctypes.byref(p), FAKE_OUT, cap, 0, WS + 128, wsb, 0) == zc.ZC_ERR_MISALIGNED
    assert st(FAKE_IN, n, ctypes.byref(p), FAKE_OUT, cap, 0, WS, wsb - 1, 0) == zc.ZC_ERR_CAPACITY
    assert st(FAKE_IN, n, ctypes.byref(p), FAKE_OUT, cap - 1, 0, WS, wsb, 0) == zc.ZC_ERR_CAPACITY
    assert st(FAKE_IN + 2, n, ctypes.byref(p), FAKE_OUT, cap, 0, WS, wsb, 0) == zc.ZC_ERR_MISALIGNED
    arr, k = zc.make_enc_segs([(FAKE_IN, n, PLAN, FAKE_OUT, cap, 0), (FAKE_IN, 5000, PLAN, FAKE_OUT + (1 << 20),
                                                                      zc.zc_max_compressed_bytes(5000), 0)])
    need = wsb + zc.zc_compress_workspace_bytes(5000)
    assert zc.raw_status("zc_compress_batch_ws", arr, k, WS, need - 256, 0) == zc.ZC_ERR_CAPACITY
    assert zc.raw_status("zc_compress_batch_ws", arr, k, 0, need, 0) == zc.ZC_ERR_INVALID_ARG
    # without a workspace the same output buffers are too small (the scratch goes behind the stream)
    assert zc.raw_status("zc_compress_batch", arr, k, 0) == zc.ZC_ERR_CAPACITY


def test_decompress_host_errors(zc):
    n = 1000
    smallest = oracle.layout(n)["off_zp"]
    st = lambda *a: zc.raw_status("zc_decompress", *a)
    assert st(FAKE_OUT, smallest - 1, n, FAKE_IN, 0, 0) == zc.ZC_ERR_CORRUPT
    assert st(0, 1 << 20, n, FAKE_IN, 0, 0) == zc.ZC_ERR_INVALID_ARG
    assert st(FAKE_OUT, 1 << 20, n, 0, 0, 0) == zc.ZC_ERR_INVALID_ARG
    assert st(FAKE_OUT, 1 << 20, 1 << 32, FAKE_IN, 0, 0) == zc.ZC_ERR_INVALID_ARG
    assert st(FAKE_OUT + 16, 1 << 20, n, FAKE_IN, 0, 0) == zc.ZC_ERR_MISALIGNED
    assert st(FAKE_OUT, 1 << 20, n, FAKE_IN + 8, 0, 0) == zc.ZC_ERR_MISALIGNED
    assert st(FAKE_OUT, 1 << 20, n, FAKE_IN, FAKE_IN + 2, 0) == zc.ZC_ERR_MISALIGNED


def test_library_histogram_plan_equals_oracle(zc):
    rng = np.random.default_rng(17)
    cases = [np.zeros(256, np.uint64), np.full(256, 3, np.uint64)]
    for trial in range(300):
        h = rng.integers(0, 5, 256).astype(np.uint64)
        if trial % 3 == 0:
            h[rng.integers(0, 256, 9)] += np.uint64(rng.integers(1, 1 << 52))  # the oracle is exact below 2^53
        cases.append(h)
    x = workloads.bf16_bits_from_f32((rng.standard_normal(100_000) * 0.02).astype(np.float32))
    cases.append(oracle.exponent_histogram(x))
    for h in cases:
        assert zc.zc_plan_from_histogram(h) == oracle.plan_from_histogram(h)
    assert zc.raw_status("zc_plan_from_histogram", None, ctypes.byref(zc.zc_plan())) == zc.ZC_ERR_INVALID_ARG
    assert zc.raw_status("zc_plan_from_histogram", (ctypes.c_uint64 * 256)(), None) == zc.ZC_ERR_INVALID_ARG


def test_stats_host_errors(zc):
    ws = zc.zc_stats_workspace_bytes(1 << 28)
    assert ws > 0 and zc.zc_stats_workspace_bytes(1 << 32) == 0
    assert zc.zc_stats_workspace_bytes(0) == ws  # the workspace does not depend on n
    FAKE_WS, FAKE_H = 0x7F2000000000, 0x7F3000000000
    for fn, extra in (("zc_exponent_histogram", ()), ("zc_estimate_sigma", (0,))):
        st = lambda d_in, n, w, wb, out, *more: zc.raw_status(fn, d_in, n, w, wb, out, *(more or extra), 0)
        assert st(FAKE_IN, 1000, FAKE_WS, ws - 1, FAKE_H) == zc.ZC_ERR_CAPACITY
        assert st(0, 1000, FAKE_WS, ws, FAKE_H) == zc.ZC_ERR_INVALID_ARG
        assert st(FAKE_IN, 1000, 0, ws, FAKE_H) == zc.ZC_ERR_INVALID_ARG
        assert st(FAKE_IN, 1000, FAKE_WS, ws, 0) == zc.ZC_ERR_INVALID_ARG
        assert st(FAKE_IN, 1 << 32, FAKE_WS, ws, FAKE_H) == zc.ZC_ERR_INVALID_ARG
        assert st(FAKE_IN + 2, 1000, FAKE_WS, ws, FAKE_H) == zc.ZC_ERR_MISALIGNED
        assert st(FAKE_IN, 1000, FAKE_WS + 8, ws, FAKE_H) == zc.ZC_ERR_MISALIGNED
        assert st(FAKE_IN, 1000, FAKE_WS, ws, FAKE_H + 4) == zc.ZC_ERR_MISALIGNED
    assert zc.raw_status("zc_estimate_sigma", FAKE_IN, 1000, FAKE_WS, ws, FAKE_H, FAKE_H + 12, 0) == \
        zc.ZC_ERR_MISALIGNED


def test_read_header_of_oracle_streams(zc):
    g = np.random.default_rng(1)
    for n in (0, 5, 4096, 10_001):
        x = workloads.bf16_bits_from_f32((g.standard_normal(n) * 0.3).astype(np.float32))
        exps = oracle.plan_from_sigma(0.3)
        s = oracle.encode(x, exps)
        info = zc.zc_read_header(s[:128].tobytes())
        E = int(np.isin(oracle_pins.exponent_field(x), exps, invert=True).sum())
        assert info == {"n": n, "zero_points": E, "total_bytes": s.size,
                        "groups": (n + 4095) // 4096, "plan": exps, "raw": False}
        for pos in (0, 4, 16, 20, 25, 31, 33, 41, 100):
            bad = s[:128].copy()
            bad[pos] ^= 0x40
            with pytest.raises(zc.ZcError):
                zc.zc_read_header(bad.tobytes())
        # a changed n may still describe a self-consistent stream; the decoder
        # compares it with the caller's n, the parser reports it
        bad = s[:128].copy()
        bad[8] ^= 0x40
        try:
            assert zc.zc_read_header(bad.tobytes())["n"] != n
        except zc.ZcError:
            pass
    with pytest.raises(zc.ZcError):
        zc.zc_read_header(bytes(64))


def test_read_header_of_raw_streams(zc):
    for n, E in ((0, 0), (100, 3), (10_000, 10_000)):
        x = oracle_pins.with_escapes(n, E, 2)
        s = oracle.encode(x, oracle_pins.WINDOW_PLAN, raw_fallback=True)
        assert s.size == 128 + 2 * n
        info = zc.zc_read_header(s[:128].tobytes())
        assert info == {"n": n, "zero_points": E, "total_bytes": 128 + 2 * n,
                        "groups": (n + 4095) // 4096, "plan": oracle_pins.WINDOW_PLAN, "raw": True}
        for pos, val in ((31, 2), (31, 0), (40, s[40] ^ 4), (90, 1)):
            bad = s[:128].copy()
            bad[pos] = val
            with pytest.raises(zc.ZcError):
                zc.zc_read_header(bad.tobytes())


def test_status_strings(zc):
    for code in range(6):
        assert zc.zc_status_string(code)
    assert zc.zc_status_string(99) == "unknown status"


def test_product_never_touches_the_oracle():
    """The package (binding, build script, kernels) neither imports nor links
    nor loads anything under oracle/: the oracle is test infrastructure only."""
    pkg = os.path.join(ROOT, "lossless_bf16_exponent_amd")
    pattern = re.compile(r"^\s*(?:import|from)\s+oracle\b|liboracle|zc_oracle|oracle/|#\s*include\s*\"[^\"]*oracle",
                         re.M)
    for dirpath, _, files in os.walk(pkg):
        for name in files:
            if name.endswith((".py", ".hip", ".h", ".cpp", ".c")):
                text = open(os.path.join(dirpath, name), encoding="utf-8").read()
                assert not pattern.search(text), os.path.join(dirpath, name)
    assert not any("oracle" in part for part in _build.compile_command("x.so"))
