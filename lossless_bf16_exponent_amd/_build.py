"""Compile the HIP codec library in-tree for gfx950 (hipcc cross-compiles without a GPU)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzc.so")
SOURCES = [os.path.join(CSRC, f) for f in ("zc_compress.hip", "zc_decode.hip", "zc_reduce.hip", "zc_stats.hip",
                                            "zc_host.cpp")]
ARCH = "gfx950"

# Packed-FP32 instructions stay disabled for every HIP translation unit.
HIP_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP codec library cannot be built")


def compile_command(out: str, extra=()) -> list:
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", out, *extra]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


BENCH_LIB = os.path.join(PKG, "libzc_bench.so")
BENCH_SOURCE = os.path.join(CSRC, "zc_bench.hip")


def build_bench(verbose: bool = False) -> str:
    """The benchmark's practical-ceiling kernels (copy and the codec's two
    access shapes), a library of their own that the codec never loads."""
    tmp = BENCH_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared", *HIP_FLAGS,
           BENCH_SOURCE, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, BENCH_LIB)
    return BENCH_LIB


TIMELINE_LIB = os.path.join(PKG, "libzc_timeline.so")


def build_timeline(verbose: bool = False) -> str:
    """The codec built with the compress kernels' per-block timeline
    (ZC_TIMELINE), for bench.py --timeline only; the codec never loads it."""
    return build_variant(TIMELINE_LIB, ["ZC_TIMELINE"], verbose)


def build_variant(path: str, defines, verbose: bool = False) -> str:
    """The library built with extra preprocessor definitions, at path."""
    tmp = path + ".tmp%d" % os.getpid()
    cmd = compile_command(tmp, extra=tuple("-D" + d for d in defines))
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, path)
    return path


GIVEUP_LIB = os.path.join(ROOT, "tests", "libzc_giveup.so")


def build_giveup(verbose: bool = False) -> str:
    """The library with a spin limit of 0, for the test of the give-up path of
    compress: every cross-workgroup wait of the compress kernel gives up at
    once, from the host's point of view exactly as a dispatch that broke
    workgroup order would.  Test infrastructure only; never loaded by the
    package."""
    return build_variant(GIVEUP_LIB, ["ZC_SPIN_LIMIT=0"], verbose)


FAIL_OTHERS_LIB = os.path.join(ROOT, "tests", "libzc_failothers.so")


def build_failothers(verbose: bool = False) -> str:
    """The library in which every compress workgroup other than a segment's
    header writer acts as if a wait had run out, while the header writer's
    own waits pass: the test that the failure mark alone invalidates the
    stream.  Test infrastructure only; never loaded by the package."""
    return build_variant(FAIL_OTHERS_LIB, ["ZC_FAIL_OTHERS=1"], verbose)


GUESS_LIBS = {"raw": os.path.join(ROOT, "tests", "libzc_guess_raw.so"),
              "coded": os.path.join(ROOT, "tests", "libzc_guess_coded.so")}


def build_guess(verbose: bool = False) -> dict:
    """Two builds whose raw-fallback compress guesses the same way for every
    flagged segment (raw, or coded) instead of sampling, so that tests reach
    both outcomes of both guesses on small inputs.  The streams must not
    depend on the guess.  Test infrastructure only."""
    build_variant(GUESS_LIBS["raw"], ["ZC_GUESS=1"], verbose)
    build_variant(GUESS_LIBS["coded"], ["ZC_GUESS=2"], verbose)
    return GUESS_LIBS


SPAN_LIBS = {"one-tile": os.path.join(ROOT, "tests", "libzc_dec_narrow.so"),
             "two-tile": os.path.join(ROOT, "tests", "libzc_dec_wide.so")}


def build_spans(verbose: bool = False) -> dict:
    """Two builds whose decoder takes one span form for launches of every size
    (one tile, or two), where the shipped one picks by the launch's size, so
    that tests reach both forms on small and ragged inputs.  Test
    infrastructure only."""
    build_variant(SPAN_LIBS["one-tile"], ["ZC_DEC_NARROW_MIN=0"], verbose)
    build_variant(SPAN_LIBS["two-tile"], ["ZC_DEC_NARROW_MIN=0xFFFFFFFFFFFFFFFFull", "ZC_DEC_NARROW_MAX=0"], verbose)
    return SPAN_LIBS


def assembly(out_path: str, source: str = SOURCES[0]) -> str:
    """Device assembly of the kernels (for inspection of the generated gfx950 code)."""
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC,
           "--cuda-device-only", "-S", source, "-o", out_path]
    subprocess.run(cmd, check=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
