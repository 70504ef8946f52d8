#!/usr/bin/env python3
"""Throughput of the BF16 exponent codec on one MI355X.

One step = compress every segment of the workload in one batched launch, then
decompress every stream in one batched launch (the whole hot path on the GPU).
The exponent tables are computed once per sigma on the host before timing, as
the pages precompute the table from sigma; their cost is reported as plan_us.

Headline workload: the 256 Mi-element gradient bucket (32 layer segments, per-
segment sigma log-uniform in [1e-5, 1e-2], 1 % exact zeros), the 256M-element
buffer the throughput target is set on.  Inputs are resident in HBM before any
timed region starts.

Timing of the headline.  Region 1: K steps back to back between two HIP events
on the launch stream and a host clock, with a device synchronize on both
sides; value = 2n bytes of uncompressed BF16 per step / the step time.
Region 2 (per call): HIP events on the same stream around K back-to-back
compress calls, then K back-to-back decompress calls; the slower call's
algorithmic bytes (2n + stream bytes) / its average duration is the roofline
figure against the 8 TB/s HBM peak.  No event sits between the two calls of a
step in region 1: on this stack an event record between dependent kernels
leaves the GPU idle for about 10 us.

Every workload of the pages' configurations (1, 2, 3, 4, 5a, 5b) also gets a
record: compress, decompress and checked decompress (with status words, the
form a collective uses) timed in R groups of back-to-back calls (each group
at least 1 ms of calls, behind an untimed lead call), mean and
p10 / p50 / p90 of the per-call time over the groups, HBM fraction, bits per
value; the two cache-resident configurations (1, 2) also cold, rotating
through enough buffer sets that the footprint exceeds the 256 MB MALL twice.
Then the one-GPU parts of the collectives: the all-gather receive side
(7 peer shards of 4096 x 14336 decoded in one batched launch into one
gathered buffer), the all-to-all order (static segments in one launch, then
the dynamic ones), the reduce-scatter receive side (decode + float32
accumulate), the plan variants (histogram, sigma estimate) and the raw
fallback; the practical ceilings of the codec's access shapes (a bench-only
library); and the CPU oracle on the host cores (one thread, and all cores).

Printed: one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = "lossless_bf16_exponent_amd/csrc/"
_COMMON = [_CSRC + f for f in ("zc_device.h", "zc_lane.h", "zc_format.h")]
# the sources each call's kernels are built from: a counter summary of a call
# is used only while these are unchanged
CALL_SOURCES = {"compress": [_CSRC + "zc_compress.hip", _CSRC + "zc_grid.h"] + _COMMON,
                "decompress": [_CSRC + "zc_decode.hip"] + _COMMON,
                "reduce": [_CSRC + "zc_reduce.hip"] + _COMMON,
                "stats": [_CSRC + "zc_stats.hip"] + _COMMON}
MALL_BYTES = 256 << 20
GROUPS = 10  # timing groups per call kind in the per-workload records
BOX_CORES = 16  # the host cores of one GPU's share on the MI355X boxes


def log(msg: str) -> None:
    print("# " + msg, file=sys.stderr, flush=True)


def kernel_source_hash(call: str) -> str:
    """Hash of the sources of one call's kernels (CALL_SOURCES): a counter
    summary is used only while the kernels it measured are unchanged."""
    h = hashlib.sha256()
    for rel in CALL_SOURCES[call]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(call: str, workload: str):
    """HBM bytes per call from the committed rocprofv3 counter summary, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(PROFILES, "traffic_%s_%s.txt" % (call, workload))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_sha") != kernel_source_hash(call):
        return None
    try:
        return int(float(vals["fetch_bytes"]) + float(vals["write_bytes"]))
    except (KeyError, ValueError):
        return None


def pct(vals, q):
    import numpy as np
    return float(np.percentile(np.asarray(vals, dtype=np.float64), q))


MIN_GROUP_US = 1000.0  # GPU time a timing group spans at least


def timed_groups(call, stream, groups: int, per: int) -> list:
    """Per-call microseconds of `groups` groups of back-to-back calls (HIP
    events on the launch stream around each group).  A group holds `per`
    calls, or more where that spans less than MIN_GROUP_US (the count is
    taken from a first, untimed group).  Each group starts behind one untimed
    lead call, so the device is busy when the start event is recorded: the
    host's launch time after the previous synchronize falls outside the timed
    region, as it does for calls queued behind other work."""
    import math
    import torch

    def group(k: int) -> float:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        call()
        e0.record(stream)
        for _ in range(k):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / k

    per = max(per, int(math.ceil(MIN_GROUP_US / max(group(per), 1e-3))))
    return [group(per) for _ in range(groups)]


def summary(us: list, alg_bytes: int, n: int) -> dict:
    mean = sum(us) / len(us)
    return {"us": round(mean, 2), "p10_us": round(pct(us, 10), 2), "p50_us": round(pct(us, 50), 2),
            "p90_us": round(pct(us, 90), 2), "uncompressed_gbps": round(2.0 * n / (mean * 1e-6) / 1e9, 1),
            "hbm_frac": round(alg_bytes / (mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}


class Resident:
    """One workload resident on the GPU: input, output slots (one per segment,
    zc_max_compressed_bytes each: the stream bound), the encoder's workspace
    (reused by every compress call), sizes, decode buffer and status words,
    with the batched segment arrays for compress, decompress and checked
    decompress."""

    def __init__(self, zc, w, x=None):
        import numpy as np
        import torch
        self.w = w
        self.plans = [zc.zc_plan_from_sigma(seg.sigma) for seg in w.segments]
        self.x = x if x is not None else torch.from_numpy(w.buffer.view(np.int16)).cuda()
        self.ns = [seg.x.size for seg in w.segments]
        offs = np.concatenate([[0], np.cumsum(self.ns)]).astype(np.int64)
        caps = [zc.zc_max_compressed_bytes(n) for n in self.ns]
        slots = [(c + 255) // 256 * 256 for c in caps]
        soff = np.concatenate([[0], np.cumsum(slots)]).astype(np.int64)
        self.out = torch.empty(int(soff[-1]), dtype=torch.uint8, device="cuda")
        self.sizes = torch.zeros(len(self.ns), dtype=torch.int64, device="cuda")
        self.dec = torch.empty_like(self.x)
        self.status = torch.zeros(len(self.ns), dtype=torch.int32, device="cuda")
        xb, ob, db = self.x.data_ptr(), self.out.data_ptr(), self.dec.data_ptr()
        ns = self.ns
        self.offs, self.soff, self.caps = offs, soff, caps
        self.enc = zc.make_enc_segs([(xb + 2 * int(offs[i]) if ns[i] else 0, ns[i], self.plans[i],
                                      ob + int(soff[i]), caps[i], self.sizes.data_ptr() + 8 * i)
                                     for i in range(len(ns))])
        self.dec_segs = zc.make_dec_segs([(ob + int(soff[i]), caps[i], ns[i], db + 2 * int(offs[i]) if ns[i] else 0, 0)
                                          for i in range(len(ns))])
        self.chk_segs = zc.make_dec_segs([(ob + int(soff[i]), caps[i], ns[i], db + 2 * int(offs[i]) if ns[i] else 0,
                                           self.status.data_ptr() + 4 * i) for i in range(len(ns))])
        self.ws = torch.empty(sum(zc.zc_compress_workspace_bytes(n) for n in ns), dtype=torch.uint8, device="cuda")
        self.footprint = self.x.numel() * 2 + self.out.numel() + self.dec.numel() * 2 + self.ws.numel()

    def compress(self, zc, stream, segs=None) -> None:
        """One batched compress with the scratch in the workspace."""
        zc.zc_compress_batch_ws(self.enc if segs is None else segs, self.ws, self.ws.numel(), stream)

    def check(self, zc, stream) -> dict:
        """One checked round trip; returns the stream facts."""
        import torch
        self.status.fill_(-1)
        self.compress(zc, stream)
        zc.zc_decompress_batch(self.chk_segs, stream)
        torch.cuda.synchronize()
        if self.status.any() or not torch.equal(self.dec, self.x):
            raise RuntimeError("GPU round trip is not lossless on %s" % self.w.name)
        totals = [int(v) for v in self.sizes.cpu()]
        zero_points, raw = 0, 0
        for i in range(len(self.ns)):
            o = int(self.soff[i])
            hdr = self.out[o:o + 40].cpu().numpy().tobytes()
            zero_points += int.from_bytes(hdr[32:40], "little")
            raw += hdr[31] == 1
        return {"stream_bytes": sum(totals), "zero_points": zero_points, "raw_segments": raw}


def measure_workload(zc, w, steps: int, warmup: int, cold: bool = False) -> dict:
    """The record of one workload: compress, decompress and checked decompress
    in GROUPS groups of back-to-back calls; cold: also with buffer sets rotated
    so that no call finds its input in the MALL."""
    import torch
    stream = torch.cuda.current_stream()
    r = Resident(zc, w)
    facts = r.check(zc, stream)
    n = w.n
    alg = 2 * n + facts["stream_bytes"]
    per = max(1, steps // GROUPS)
    rec = {"workload": w.name, "values": n, "segments": len(w.segments), "stream_bytes": facts["stream_bytes"],
           "bits_per_value": round(8.0 * facts["stream_bytes"] / n, 4),
           "compression_ratio": round(facts["stream_bytes"] / (2.0 * n), 5),
           "zero_point_rate": round(facts["zero_points"] / n, 6), "algorithmic_bytes_per_call": int(alg),
           "timing": "%d groups of back-to-back calls (at least %d and at least %g us of calls per group, each "
                     "behind an untimed lead call) after %d warm-up calls; mean and percentiles of the per-call "
                     "time over the groups" % (GROUPS, per, MIN_GROUP_US, warmup)}
    calls = {"compress": lambda: r.compress(zc, stream),
             "decompress": lambda: zc.zc_decompress_batch(r.dec_segs, stream),
             "decompress_checked": lambda: zc.zc_decompress_batch(r.chk_segs, stream)}
    for name, call in calls.items():
        for _ in range(warmup):
            call()
        rec[name] = summary(timed_groups(call, stream, GROUPS, per), alg, n)
    rec["decompress_checked"]["kernels"] = "zero_kernel (status words) + decode_kernel"
    for name in ("compress", "decompress"):
        t = load_traffic(name, w.name)  # counter bytes per call, when profiled for the current kernels
        rec[name]["traffic"] = t
        rec[name]["traffic_over_algorithmic"] = round(t / alg, 4) if t else None
    if not torch.equal(r.dec, r.x):
        raise RuntimeError("decoded buffer differs after timing on %s" % w.name)
    if cold:
        sets = [r] + [Resident(zc, w, x=r.x.clone()) for _ in range(max(1, 2 * MALL_BYTES // r.footprint))]
        for s in sets[1:]:
            s.check(zc, stream)
        k = len(sets)
        rec["cache_resident"] = True
        rec["cold"] = {"buffer_sets": k, "footprint_bytes": int(sum(s.footprint for s in sets))}
        for name, attr in (("compress", "enc"), ("decompress", "dec_segs")):
            fns = [(lambda s=s, a=attr: s.compress(zc, stream) if a == "enc" else zc.zc_decompress_batch(
                getattr(s, a), stream)) for s in sets]
            it = [0]

            def rot():
                fns[it[0] % k]()
                it[0] += 1
            for _ in range(k):
                rot()
            rec["cold"][name] = summary(timed_groups(rot, stream, GROUPS, max(per, k)), alg, n)
        del sets
    del r
    torch.cuda.empty_cache()
    return rec


def allgather_receive(zc, steps: int, warmup: int) -> dict:
    """The one-GPU part of a compressed all-gather of Llama3-8B shards over 8
    ranks: this rank's 4096 x 14336 shard compressed once, and the 7 peers'
    streams decoded in one batched launch into one gathered buffer.  Peer p's
    shard is N(0, 0.02^2), drawn on the device from a seeded generator and
    rounded to BF16 (nearest even), compressed untimed."""
    import torch
    stream = torch.cuda.current_stream()
    shard, peers = 4096 * 14336, 7
    plan = zc.zc_plan_from_sigma(0.02)
    gathered = torch.empty(peers * shard, dtype=torch.int16, device="cuda")
    src = torch.empty_like(gathered)
    for p in range(peers):
        g = torch.Generator(device="cuda").manual_seed(100 + p)
        src[p * shard:(p + 1) * shard] = (torch.randn(shard, generator=g, device="cuda") * 0.02).to(
            torch.bfloat16).view(torch.int16)
    cap = zc.zc_max_compressed_bytes(shard)
    slot = (cap + 255) // 256 * 256
    bufs = torch.empty(peers * slot, dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(peers, dtype=torch.int64, device="cuda")
    enc = zc.make_enc_segs([(src.data_ptr() + 2 * p * shard, shard, plan, bufs.data_ptr() + p * slot, cap,
                             sizes.data_ptr() + 8 * p) for p in range(peers)])
    ws = torch.empty(peers * zc.zc_compress_workspace_bytes(shard), dtype=torch.uint8, device="cuda")
    zc.zc_compress_batch_ws(enc, ws, ws.numel(), stream)
    torch.cuda.synchronize()
    totals = [int(v) for v in sizes.cpu()]
    dec = zc.make_dec_segs([(bufs.data_ptr() + p * slot, totals[p], shard, gathered.data_ptr() + 2 * p * shard, 0)
                            for p in range(peers)])
    zc.zc_decompress_batch(dec, stream)
    torch.cuda.synchronize()
    if not torch.equal(gathered, src):
        raise RuntimeError("all-gather receive side is not lossless")
    per = max(1, steps // GROUPS)
    alg = sum(totals) + 2 * peers * shard
    call = lambda: zc.zc_decompress_batch(dec, stream)
    for _ in range(warmup):
        call()
    rec = {"peers": peers, "shard_values": shard, "stream_bytes": sum(totals),
           "decompress_gathered": summary(timed_groups(call, stream, GROUPS, per), alg, peers * shard)}
    one = zc.make_enc_segs([(src.data_ptr(), shard, plan, bufs.data_ptr(), cap, sizes.data_ptr())])
    call = lambda: zc.zc_compress_batch_ws(one, ws, ws.numel(), stream)
    for _ in range(warmup):
        call()
    rec["compress_own_shard"] = summary(timed_groups(call, stream, GROUPS, per), 2 * shard + totals[0], shard)
    rec["kernels"] = {"decompress_gathered": "decode_kernel, 7 segments in one launch",
                      "compress_own_shard": "compress_kernel"}
    del gathered, src, bufs, ws
    torch.cuda.empty_cache()
    return rec


def alltoall_order(zc, w, steps: int, warmup: int) -> dict:
    """The all-to-all segments of one rank (workload 4) in the two-phase order
    the pages describe: the 8 static (fixed-size) segments compressed in one
    launch, then the 8 dynamic ones in a second launch, back to back; against
    all 16 in one launch."""
    import torch
    stream = torch.cuda.current_stream()
    r = Resident(zc, w)
    facts = r.check(zc, stream)
    ns, plans = r.ns, r.plans
    xb, ob = r.x.data_ptr(), r.out.data_ptr()

    def segs(idx):
        return zc.make_enc_segs([(xb + 2 * int(r.offs[i]) if ns[i] else 0, ns[i], plans[i], ob + int(r.soff[i]),
                                  r.caps[i], r.sizes.data_ptr() + 8 * i) for i in idx])
    static, dynamic = segs(range(8)), segs(range(8, 16))
    per = max(1, steps // GROUPS)
    alg = 2 * w.n + facts["stream_bytes"]
    # (one workspace for both launches: calls on one stream may share it)
    two = lambda: (r.compress(zc, stream, static), r.compress(zc, stream, dynamic))
    one = lambda: r.compress(zc, stream)
    rec = {}
    for name, call in (("static_then_dynamic", two), ("one_launch", one)):
        for _ in range(warmup):
            call()
        rec[name] = summary(timed_groups(call, stream, GROUPS, per), alg, w.n)
    rec["launches"] = {"static_then_dynamic": 2, "one_launch": 1}
    del r
    torch.cuda.empty_cache()
    return rec


TIMELINE_WORDS = 5  # per block in the instrumented build: four clock stamps and the role
TIMELINE_TICK_US = 0.01  # the real-time clock runs at 100 MHz


def timeline(zc, w, warmup: int, burst: int = 1) -> dict:
    """Per-block timeline of one batched compress of workload w (no raw
    fallback), from the instrumented build (libzc_timeline.so, ZC_TIMELINE):
    after `warmup` calls, `burst` back-to-back calls (HIP events between them)
    with every block's four clock stamps and role recorded (stamp meanings in
    zc_compress.hip); the stamps are the last call's, each call overwriting
    the previous one's.  burst = 1: one call right after a synchronize; a
    longer burst gives the steady state of back-to-back calls.  The record
    gives, per role, the median time between stamps, and the launch's tail:
    what ends after the last encoder block."""
    import ctypes
    import numpy as np
    import torch
    from lossless_bf16_exponent_amd import _build
    lib = ctypes.CDLL(_build.TIMELINE_LIB)
    lib.zc_compress_batch_ws.argtypes = [ctypes.POINTER(zc.zc_enc_seg), ctypes.c_uint32, ctypes.c_void_p,
                                         ctypes.c_uint64, ctypes.c_void_p]
    lib.zc_compress_batch_ws.restype = ctypes.c_int
    lib.zc_timeline_clear.restype = ctypes.c_int
    lib.zc_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
    lib.zc_timeline_read.restype = ctypes.c_int
    stream = torch.cuda.current_stream()
    r = Resident(zc, w)
    arr, k = r.enc

    def call():
        rc = lib.zc_compress_batch_ws(arr, k, r.ws.data_ptr(), r.ws.numel(), stream.cuda_stream)
        if rc != zc.ZC_OK:
            raise RuntimeError("instrumented compress failed: %d" % rc)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    if lib.zc_timeline_clear() != 0:
        raise RuntimeError("zc_timeline_clear failed")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(max(1, burst) + 1)]
    ev[0].record(stream)
    for i in range(max(1, burst)):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    e0, e1 = ev[-2], ev[-1]
    buf = np.zeros(TIMELINE_WORDS << 20, dtype=np.uint64)
    if lib.zc_timeline_read(buf.ctypes.data, buf.nbytes) != 0:
        raise RuntimeError("zc_timeline_read failed")
    t = buf.reshape(-1, TIMELINE_WORDS)
    ran = np.flatnonzero(t[:, 0])
    blocks = int(ran.max()) + 1
    t = t[:blocks]
    stamps = t[:, :4].astype(np.int64)
    stamps = (stamps - stamps[:, 0].min()) * TIMELINE_TICK_US
    role = t[:, 4].astype(np.int64)
    kind, seg = role & 3, (role >> 2) & 63
    names = {0: "encoder_staged", 1: "encoder_direct", 2: "finalize"}

    def med(a):
        return round(float(np.median(a)), 2) if a.size else None
    rec = {"workload": w.name, "values": w.n, "burst": max(1, burst),
           "event_us": round(e0.elapsed_time(e1) * 1e3, 2), "blocks": blocks,
           "span_us": round(float(stamps[:, 3].max()), 2), "stamps": "0 start, 1 first pass or span words, "
           "2 bytes staged or offset known, 3 end (zc_compress.hip)", "roles": {}}
    for kd, name in names.items():
        m = kind == kd
        if not m.any():
            continue
        S = stamps[m]
        rec["roles"][name] = {"blocks": int(m.sum()), "lifetime_median_us": med(S[:, 3] - S[:, 0]),
                              "stamp_0_1_median_us": med(S[:, 1] - S[:, 0]),
                              "stamp_1_2_median_us": med(S[:, 2] - S[:, 1]),
                              "stamp_2_3_median_us": med(S[:, 3] - S[:, 2]),
                              "last_start_us": round(float(S[:, 0].max()), 2),
                              "last_end_us": round(float(S[:, 3].max()), 2)}
    enc = kind < 2
    last_enc = float(stamps[enc, 3].max())
    late = stamps[:, 3] > last_enc
    rec["tail"] = {"last_encoder_end_us": round(last_enc, 2), "blocks_ending_later": int(late.sum()),
                   "segments": sorted(set(int(v) for v in seg[late])), "last_end_us": round(float(stamps[:, 3].max()), 2)}
    last = int(np.argmax(stamps[:, 3]))
    rec["tail"]["last_block"] = {"role": names.get(int(kind[last]), str(int(kind[last]))), "segment": int(seg[last]),
                                 "stamps_us": [round(float(v), 2) for v in stamps[last]]}
    del r
    torch.cuda.empty_cache()
    return rec


def profile_pass(zc, w, call: str, steps: int) -> dict:
    """The command rocprofv3 counter passes run (--profile CALL): a copy of
    known size with the bench library's copy kernel (the counters' scale: the
    bytes the copy reads and writes over what the counters report), then
    `steps` calls of CALL on workload w as the bench times them (compress and
    decompress on the resident workload; reduce on the 32 Mi-value shard of 7
    peers)."""
    import torch
    from lossless_bf16_exponent_amd import _build
    lib = ctypes.CDLL(_build.BENCH_LIB)
    vp, u64 = ctypes.c_void_p, ctypes.c_uint64
    lib.zcb_copy.argtypes = [vp, vp, u64, vp]
    stream = torch.cuda.current_stream()
    copy_bytes = 1 << 30
    a = torch.full((copy_bytes // 2,), 0x3C00, dtype=torch.int16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        if lib.zcb_copy(a.data_ptr(), b.data_ptr(), copy_bytes, stream.cuda_stream) != 0:
            raise RuntimeError("copy kernel failed")
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()
    rec = {"profile": call, "copy_kernel_bytes": copy_bytes, "steps": steps}
    if call == "reduce":
        rec["reduce"] = reduce_measurement(zc, steps)
        return rec
    r = Resident(zc, w)
    facts = r.check(zc, stream)
    fn = (lambda: r.compress(zc, stream)) if call == "compress" else (lambda: zc.zc_decompress_batch(r.dec_segs, stream))
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    rec.update({"workload": w.name, "values": w.n, "stream_bytes": facts["stream_bytes"],
                "algorithmic_bytes_per_call": 2 * w.n + facts["stream_bytes"]})
    return rec


def ceilings(n: int, steps: int, warmup: int) -> dict:
    """Practical ceilings of the codec's access shapes for n values (a
    bench-only library): a 128-bit copy of 2n bytes, the encoder's shape (read
    2 B, write 1.375 B per value) and the decoder's (read 1.375 B, write 2 B),
    each timed after `warmup` calls like the codec's own calls."""
    import torch
    from lossless_bf16_exponent_amd import _build
    lib = ctypes.CDLL(_build.BENCH_LIB)
    vp, u64 = ctypes.c_void_p, ctypes.c_uint64
    lib.zcb_copy.argtypes = [vp, vp, u64, vp]
    lib.zcb_encode_shape.argtypes = [vp, u64, vp, vp, vp]
    lib.zcb_decode_shape.argtypes = [vp, vp, u64, vp, vp]
    stream = torch.cuda.current_stream()
    st = stream.cuda_stream
    a = torch.empty(n, dtype=torch.int16, device="cuda")
    b = torch.empty(n, dtype=torch.int16, device="cuda")
    sm = torch.empty(n, dtype=torch.uint8, device="cuda")
    pl = torch.empty(3 * n // 8, dtype=torch.uint8, device="cuda")
    a.fill_(0x3C00)
    calls = {"copy": (lambda: lib.zcb_copy(a.data_ptr(), b.data_ptr(), 2 * n, st), 4 * n),
             "encode_shape": (lambda: lib.zcb_encode_shape(a.data_ptr(), n, sm.data_ptr(), pl.data_ptr(), st),
                              2 * n + n + 3 * n // 8),
             "decode_shape": (lambda: lib.zcb_decode_shape(sm.data_ptr(), pl.data_ptr(), n, b.data_ptr(), st),
                              2 * n + n + 3 * n // 8)}
    rec = {"values": n, "library": "libzc_bench.so (bench only)"}
    for name, (call, nbytes) in calls.items():
        for _ in range(warmup):
            if call() != 0:
                raise RuntimeError("ceiling kernel %s failed" % name)
        us = timed_groups(call, stream, 5, max(1, steps // 5))
        mean = sum(us) / len(us)
        rec[name] = {"us": round(mean, 2), "bytes": int(nbytes), "gbps": round(nbytes / (mean * 1e-6) / 1e9, 1),
                     "hbm_frac": round(nbytes / (mean * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
    # torch's own device-to-device copy, for reference
    for _ in range(warmup):
        b.copy_(a)
    us = timed_groups(lambda: b.copy_(a), stream, 5, max(1, steps // 5))
    mean = sum(us) / len(us)
    rec["torch_copy"] = {"us": round(mean, 2), "bytes": 4 * n, "gbps": round(4 * n / (mean * 1e-6) / 1e9, 1)}
    del a, b, sm, pl
    torch.cuda.empty_cache()
    return rec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, plans, one_thread_segments: int = 8, min_seconds: float = 5.0, max_passes: int = 6) -> dict:
    """The oracle as it stands (plain C -O2, unchanged), timed on the host:
    on one thread over the first segments, and on all the host cores this
    GPU's share has (a thread pool over all segments; ctypes releases the GIL
    during each call), each repeated to about min_seconds."""
    import numpy as np
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    segs = list(zip(w.segments, plans))
    outs = [np.empty(oracle.max_bytes(seg.x.size), dtype=np.uint8) for seg, _ in segs]
    decs = [np.empty(seg.x.size, dtype=np.uint16) for seg, _ in segs]

    def one(i):
        seg, plan = segs[i]
        t0 = time.perf_counter()
        total = oracle.encode_into(seg.x, plan, outs[i])
        t1 = time.perf_counter()
        rc = oracle.decode_into(outs[i][:total], seg.x.size, decs[i])
        t2 = time.perf_counter()
        if rc != 0 or not np.array_equal(decs[i], seg.x):
            raise RuntimeError("oracle round trip failed on the CPU sample")
        return t1 - t0, t2 - t1

    # one thread
    k1 = min(one_thread_segments, len(segs))
    n1 = sum(segs[i][0].x.size for i in range(k1))
    t_enc = t_dec = 0.0
    passes = 0
    while passes < max_passes and (passes == 0 or t_enc + t_dec < min_seconds):
        for i in range(k1):
            a, b = one(i)
            t_enc += a
            t_dec += b
        passes += 1
    gb1 = 2.0 * n1 * passes / 1e9
    single = {"value": round(gb1 / (t_enc + t_dec), 4), "unit": "GB/s", "cores": 1,
              "compress_gbps": round(gb1 / t_enc, 4), "decompress_gbps": round(gb1 / t_dec, 4),
              "sample": "first %d of %d segments (%d BF16 values), compress + decompress, %d pass(es)"
                        % (k1, len(segs), n1, passes)}
    # all cores of the share
    affinity = len(os.sched_getaffinity(0))
    threads = max(1, min(affinity, BOX_CORES, len(segs)))
    n = sum(seg.x.size for seg, _ in segs)
    passes = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_seconds):
            list(ex.map(one, range(len(segs))))
            passes += 1
    wall = time.perf_counter() - t0
    gb = 2.0 * n * passes / 1e9
    return {"value": round(gb / wall, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "all %d segments (%d BF16 values) of the workload, compress + decompress of each, %d pass(es), "
                      "%d threads each running the unchanged plain C -O2 oracle on whole segments"
                      % (len(segs), n, passes, threads),
            "seconds": round(wall, 3), "affinity_cpus": affinity, "cpu_model": cpu_model(),
            "single_thread": single}


REDUCE_WARMUP_CALLS = 300


def reduce_measurement(zc, steps: int) -> dict:
    """The receive side of a reduce-scatter run as a zipped all-to-all (section
    2.D): one rank's 32 Mi-value shard, compressed contributions of 7 peers
    plus the local share, reduced by zc_decompress_reduce.  Peer p's values are
    N(0, sigma_p^2) with sigma_p the first eight layer sigmas of the gradient
    bucket, each compressed with its own plan.  HIP events around K calls,
    after REDUCE_WARMUP_CALLS calls: per-call timings of 1,000 calls in a row on
    MI355X, in means over 50 calls, go 111, 99, 93, 89, 87, 86 us and then stay
    at 85-86 us from about the 250th call on (the device settling after a burst
    of this kernel), the steady state a training job that reduces bucket after
    bucket sees."""
    import torch

    call, state = reduce_setup(zc)
    n, peers, totals = state["n"], state["peers"], state["totals"]
    stream = torch.cuda.current_stream()
    for _ in range(REDUCE_WARMUP_CALLS):
        call()
    torch.cuda.synchronize()
    alg = sum(totals) + 4 * n  # the peer streams and the local share read, the result written
    us = timed_groups(call, stream, GROUPS, max(1, steps // GROUPS))
    rec = summary(us, alg, n)
    t = load_traffic("reduce", "shard-32M-7peers")
    rec.update({"traffic": t, "traffic_over_algorithmic": round(t / alg, 4) if t else None})
    rec.update({"shard_values": n, "peers": peers, "local": True, "warmup_calls": REDUCE_WARMUP_CALLS,
                "uncompressed_gbps": round(2.0 * n * (peers + 1) / (rec["us"] * 1e-6) / 1e9, 1),
                "algorithmic_bytes": int(alg), "achieved_gbps": round(alg / (rec["us"] * 1e-6) / 1e9, 1),
                "kernel": "reduce_kernel"})
    del state
    torch.cuda.empty_cache()
    return rec


def reduce_setup(zc):
    """The shard of reduce_measurement, its 7 peers compressed: returns one
    zc_decompress_reduce call (a function) and the buffers it uses."""
    import numpy as np
    import torch

    from lossless_bf16_exponent_amd import workloads

    n, peers = 1 << 25, 7
    sig = workloads.config3_sigmas()[:peers + 1]
    g = np.random.default_rng(21)
    xs = [torch.from_numpy(workloads.bf16_bits_from_f32(g.standard_normal(n).astype(np.float32)
                                                          * np.float32(s)).view(np.int16)).cuda() for s in sig]
    cap = zc.zc_compress_capacity(n)  # (untimed setup: the scratch behind each stream)
    bufs = [torch.empty(cap, dtype=torch.uint8, device="cuda") for _ in range(peers)]
    sizes = torch.zeros(peers, dtype=torch.int64, device="cuda")
    for p in range(peers):
        zc.zc_compress(xs[p + 1], n, zc.zc_plan_from_sigma(float(sig[p + 1])), bufs[p], cap, sizes.data_ptr() + 8 * p)
    torch.cuda.synchronize()
    totals = [int(v) for v in sizes.cpu()]
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    ptrs = [b.data_ptr() for b in bufs]
    state = {"n": n, "peers": peers, "totals": totals, "xs": xs, "bufs": bufs, "out": out}
    return (lambda: zc.zc_decompress_reduce(ptrs, totals, n, xs[0], out, None, stream)), state


def percall(zc, w, call: str, calls: int) -> dict:
    """HIP-event time of every one of `calls` back-to-back calls of one kind
    (compress or decompress of workload w, or the reduce of
    reduce_measurement), from the first call of the run on: the device's
    start-of-burst transient that the warm-up counts are set from.  Means over
    blocks of 50 calls."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    keep = None
    if call == "reduce":
        fn, keep = reduce_setup(zc)
    else:
        keep = Resident(zc, w)
        keep.check(zc, stream)
        fn = (lambda: keep.compress(zc, stream)) if call == "compress" else (
            lambda: zc.zc_decompress_batch(keep.dec_segs, stream))
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
    ev[0].record(stream)
    for i in range(calls):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(calls)])
    del keep
    torch.cuda.empty_cache()
    return {"call": call, "workload": "shard-32M-7peers" if call == "reduce" else w.name, "calls": calls,
            "note": "an event recorded between two kernels adds to each call; compare the blocks with each other",
            "mean_us_per_50_calls": [round(float(t[i:i + 50].mean()), 1) for i in range(0, calls - 49, 50)]}
    return rec


def stats_measurement(zc, x, seg_ns, steps: int, warmup: int) -> dict:
    """The online statistics that section 2.A replaces by its sigma-derived
    table, on the resident gradient bucket: the exponent histogram and the
    sigma estimate of the whole buffer (HIP events around groups of back-to-back
    calls after `warmup` calls; algorithmic bytes = the 2n input bytes read), and the wall time of
    the histogram route to a table for every segment (one histogram per
    segment, one copy of the counts to the host, host top-7), against the
    closed-form route (host table from the known sigma)."""
    import numpy as np
    import torch

    n = x.numel()
    ws = torch.empty(zc.zc_stats_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    hist = torch.zeros(256, dtype=torch.int64, device="cuda")
    sig = torch.zeros(2, dtype=torch.float64, device="cuda")
    stream = torch.cuda.current_stream()
    xb = x.data_ptr()
    hist_call = lambda: zc.zc_exponent_histogram(xb, n, ws, ws.numel(), hist, stream)
    sig_call = lambda: zc.zc_estimate_sigma(xb, n, ws, ws.numel(), sig.data_ptr(), sig.data_ptr() + 8, stream)
    out = {"values": n, "kernels": {"histogram": "hist_kernel + hist_sum_kernel",
                                    "sigma": "sigma_kernel + sigma_final_kernel"}}
    for name, call in (("histogram", hist_call), ("sigma", sig_call)):
        for _ in range(warmup):
            call()
        us = timed_groups(call, stream, 5, max(1, steps // 5))
        ms = sum(us) / len(us) / 1e3
        gbps = 2.0 * n / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 2), "achieved_gbps": round(gbps, 1),
                     "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes": 2 * n}
    if int(hist.sum().item()) != n:
        raise RuntimeError("histogram does not count every value")
    out["sigma"]["finite_values"] = int(sig[1:].view(torch.int64).item())

    # the histogram route to one table per segment, host clock
    offs = np.concatenate([[0], np.cumsum(seg_ns)]).astype(np.int64)
    hs = torch.zeros((len(seg_ns), 256), dtype=torch.int64, device="cuda")
    wss = [torch.empty(zc.zc_stats_workspace_bytes(m), dtype=torch.uint8, device="cuda") for m in seg_ns]

    def route():
        for i, m in enumerate(seg_ns):
            zc.zc_exponent_histogram(xb + 2 * int(offs[i]), m, wss[i], wss[i].numel(), hs[i], stream)
        h = hs.cpu().numpy()
        return [zc.zc_plan_from_histogram(h[i]) for i in range(len(seg_ns))]
    route()
    reps = max(3, min(steps, 20))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        route()
    out["histogram_route_us_per_bucket"] = round((time.perf_counter() - t0) * 1e6 / reps, 1)
    out["histogram_route"] = ("%d segment histograms + one copy of the counts to the host + %d host top-7 tables"
                              % (len(seg_ns), len(seg_ns)))
    return out


def fallback_measurement(zc, steps: int, warmup: int) -> dict:
    """The raw fallback on the stress workload that coding expands most
    (2^24 uniformly random non-NaN/Inf BF16 patterns under the sigma = 0.02
    plan, 18.8 bits per value coded): compress with ZC_PLAN_RAW_FALLBACK and
    decompress of the raw stream, in groups of back-to-back calls after
    `warmup` calls of each."""
    import numpy as np
    import torch

    from lossless_bf16_exponent_amd import workloads

    w = workloads.get("5b")
    n = w.n
    x = torch.from_numpy(w.buffer.view(np.int16)).cuda()
    plan = zc.plan_with_raw_fallback(zc.zc_plan_from_sigma(w.segments[0].sigma))
    cap = zc.zc_max_compressed_bytes(n)
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    dec = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    ws = torch.empty(zc.zc_compress_workspace_bytes(n), dtype=torch.uint8, device="cuda")
    enc_call = lambda: zc.zc_compress_ws(x, n, plan, out, cap, size, ws, ws.numel(), stream)
    dec_call = lambda: zc.zc_decompress(out, cap, n, dec, None, stream)
    enc_call()
    dec_call()
    torch.cuda.synchronize()
    total = int(size.item())
    if total != 128 + 2 * n or out[31].item() != 1 or not torch.equal(dec, x):
        raise RuntimeError("the fallback did not give a lossless raw stream")
    res = {"workload": w.name, "values": n, "stream_bytes": total, "raw": True}
    alg = 2 * n + total
    for name, call in (("compress", enc_call), ("decompress", dec_call)):
        for _ in range(warmup):
            call()
        res[name] = summary(timed_groups(call, stream, GROUPS, max(1, steps // GROUPS)), alg, n)
    res["kernels"] = {"compress": "compress_fallback_kernel (the guessing launch) + compress_second_kernel",
                      "decompress": "decode_kernel (raw branch)"}
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # Compress calls on a fresh device run slower for their first few dozen
    # calls (device clock and power settling; measured on the bucket with
    # 5 / 30 / 100 / 200 warm-up steps: 158.7 / 152.4 / 151.0 / 151.0 us per
    # compress, decompress unchanged), so the default warm-up reaches the
    # steady state that a job compressing bucket after bucket runs in.
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps before timing starts (default 100, about 30 ms on the bucket)")
    ap.add_argument("--workload", default="3", help="headline workload id (1, 2, 3, 4, 5a, 5b); default 3")
    ap.add_argument("--only-headline", action="store_true", help="skip every record besides the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timeline", action="store_true",
                    help="print the per-block timeline of one compress call of --workload, from the instrumented "
                         "build (libzc_timeline.so), instead of the bench line")
    ap.add_argument("--percall", choices=("compress", "decompress", "reduce"),
                    help="print the HIP-event time of every one of --calls back-to-back calls of this kind (means "
                         "over 50), from the run's first call on, instead of the bench line")
    ap.add_argument("--calls", type=int, default=400, help="calls for --percall (default 400)")
    ap.add_argument("--burst", type=int, default=1,
                    help="--timeline: the stamps of the last of this many back-to-back calls (the steady state "
                         "of a burst; default 1, one call after a synchronize)")
    ap.add_argument("--profile", choices=("compress", "decompress", "reduce"),
                    help="run only what a rocprofv3 counter pass measures: a copy of known size, then --steps "
                         "calls of this kind on --workload; prints that run's facts instead of the bench line")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the codec on one GPU; runs on several GPUs are not supported "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        return 2

    import torch

    from lossless_bf16_exponent_amd import workloads, zc

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)

    t_gen = time.perf_counter()
    w = workloads.get(args.workload)
    if args.profile:
        print(json.dumps(profile_pass(zc, w, args.profile, args.steps)), flush=True)
        return 0
    if args.timeline:
        print(json.dumps(timeline(zc, w, args.warmup, args.burst)), flush=True)
        return 0
    if args.percall:
        print(json.dumps(percall(zc, w, args.percall, args.calls)), flush=True)
        return 0
    log("workload %s: %d values in %d segments, generated in %.1f s"
        % (w.name, w.n, len(w.segments), time.perf_counter() - t_gen))

    t0 = time.perf_counter()
    plans = [zc.zc_plan_from_sigma(seg.sigma) for seg in w.segments]
    plan_us = (time.perf_counter() - t0) * 1e6 / len(plans)

    r = Resident(zc, w)
    stream = torch.cuda.current_stream()
    facts = r.check(zc, stream)  # correctness of what is timed: one checked round trip first
    stream_bytes = facts["stream_bytes"]
    n = w.n
    for _ in range(args.warmup):
        r.compress(zc, stream)
        zc.zc_decompress_batch(r.dec_segs, stream)
    torch.cuda.synchronize()

    # timed region 1, the whole hot path: K steps of one batched compress and
    # one batched decompress, with nothing recorded between the launches
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    g0.record(stream)
    for _ in range(args.steps):
        r.compress(zc, stream)
        zc.zc_decompress_batch(r.dec_segs, stream)
    g1.record(stream)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    gpu_step_ms = g0.elapsed_time(g1) / args.steps

    # timed region 2, per call: HIP events on the launch stream around K
    # back-to-back compress calls, then K back-to-back decompress calls
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    for _ in range(args.steps):
        r.compress(zc, stream)
    e[1].record(stream)
    for _ in range(args.steps):
        zc.zc_decompress_batch(r.dec_segs, stream)
    e[2].record(stream)
    torch.cuda.synchronize()
    enc_ms = e[0].elapsed_time(e[1]) / args.steps
    dec_ms = e[1].elapsed_time(e[2]) / args.steps
    if not torch.equal(r.dec, r.x):
        print("bench.py: decoded buffer differs after timing", file=sys.stderr)
        return 1
    x_keep = r.x
    del r
    torch.cuda.empty_cache()

    ms_per_step = t_total * 1e3 / args.steps
    gb = 2.0 * n / 1e9
    alg = 2.0 * n + stream_bytes
    # the decoder takes one-tile spans for a launch of 2^27 values or more, else two
    calls = {"compress": (enc_ms, "compress_kernel"),
             "decompress": (dec_ms, "decode_kernel<1>" if n >= 1 << 27 else "decode_kernel<2>")}
    dom = max(calls, key=lambda k: calls[k][0])
    dom_ms, dom_kernels = calls[dom]
    achieved = alg / (dom_ms * 1e-3) / 1e9
    traffic = load_traffic(dom, w.name)

    rec = {
        "metric": "compress/decompress GB/s (uncompressed BF16) + % HBM roofline; compression ratio",
        "value": round(gb / (ms_per_step * 1e-3), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u16",
        "data": "synthetic",
        "config": {"workload": w.name, "values": n, "segments": len(w.segments), "input": "bf16",
                   "description": w.description, "launches_per_step": "1 batched compress + 1 batched decompress"},
        "compress_gbps": round(gb / (enc_ms * 1e-3), 2),
        "decompress_gbps": round(gb / (dec_ms * 1e-3), 2),
        "compress_us": round(enc_ms * 1e3, 2),
        "decompress_us": round(dec_ms * 1e3, 2),
        "compress_hbm_frac": round(alg / (enc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "decompress_hbm_frac": round(alg / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "compression_ratio": round(stream_bytes / (2.0 * n), 5),
        "bits_per_value": round(8.0 * stream_bytes / n, 4),
        "zero_point_rate": round(facts["zero_points"] / n, 6),
        "plan_us": round(plan_us, 2),
        "device": dev_name,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "call": dom, "kernels": dom_kernels, "algorithmic_bytes": int(alg),
                     "avg_launch_us": round(dom_ms * 1e3, 2)},
        "gpu_step_ms": round(gpu_step_ms, 4),
        "kernel_sha": {c: kernel_source_hash(c) for c in CALL_SOURCES},
    }
    if not args.only_headline:
        rec["plan_variants"] = stats_measurement(zc, x_keep, [seg.x.size for seg in w.segments], args.steps,
                                                 args.warmup)
        rec["plan_variants"]["sigma_table_us_per_bucket"] = round(plan_us * len(w.segments), 2)
        rec["ceilings"] = ceilings(n, args.steps, args.warmup)
    del x_keep
    torch.cuda.empty_cache()
    if not args.only_headline:
        recs = {}
        for wid in ("1", "2", "3", "4", "5a", "5b"):
            t0 = time.perf_counter()
            wl = w if wid == args.workload else workloads.get(wid)
            log("workload %s (%d values): generated in %.1f s" % (wid, wl.n, time.perf_counter() - t0))
            recs[wid] = measure_workload(zc, wl, args.steps, args.warmup, cold=wid in ("1", "2"))
            if wid == "4":
                log("all-to-all order")
                rec["alltoall_order"] = alltoall_order(zc, wl, args.steps, args.warmup)
            if wl is not w:
                del wl
        rec["workloads"] = recs
        log("all-gather receive side")
        rec["allgather_receive"] = allgather_receive(zc, args.steps, args.warmup)
        log("raw fallback")
        rec["raw_fallback"] = fallback_measurement(zc, args.steps, args.warmup)
        log("reduce-scatter receive side")
        rec["reduce_scatter_local"] = reduce_measurement(zc, args.steps)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the host")
        rec["cpu_baseline"] = cpu_baseline(w, plans)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
