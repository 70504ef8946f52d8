#!/usr/bin/env python3
"""Throughput of the BF16 exponent codec on one MI355X.

One step = compress every segment of the workload in one batched launch, then
decompress every stream in one batched launch (the whole hot path on the GPU).
The exponent tables are computed once per sigma on the host before timing, as
the pages precompute the table from sigma; their cost is reported as plan_us.

Default workload: the 256 Mi-element gradient bucket (32 layer segments, per-
segment sigma log-uniform in [1e-5, 1e-2], 1 % exact zeros), the 256M-element
buffer the throughput target is set on.  Inputs are resident in HBM before the
timed region starts.

Timing.  Region 1 (the headline): K steps back to back between two HIP events
on the launch stream and a host clock, with a device synchronize on both
sides; value = 2n bytes of uncompressed BF16 per step / the step time.
Region 2 (per call): HIP events on the same stream around K back-to-back
compress calls, then K back-to-back decompress calls; the slower call's
algorithmic bytes (2n + stream bytes) / its average duration is the roofline
figure against the 8 TB/s HBM peak.  No event sits between the two calls of a
step in region 1: on this stack an event record between dependent kernels
leaves the GPU idle for about 10 us.

Printed: one JSON line with the metric, compress and decompress rates, the
compression ratio, the roofline object (with the rocprofv3-counted HBM
traffic when the committed counter summary matches the kernel sources) and
the CPU oracle timed on the host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["lossless_bf16_exponent_amd/csrc/zc_codec.hip", "lossless_bf16_exponent_amd/csrc/zc_lane.h",
                  "lossless_bf16_exponent_amd/csrc/zc_format.h", "lossless_bf16_exponent_amd/csrc/zc_grid.h"]
STATS_SOURCES = ["lossless_bf16_exponent_amd/csrc/zc_stats.hip"]


def kernel_source_hash(sources=None) -> str:
    """Hash of the codec kernel sources (or of `sources`): a counter summary
    is used only while the kernels it measured are unchanged."""
    h = hashlib.sha256()
    for rel in (KERNEL_SOURCES if sources is None else sources):
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
    if vals.get("kernel_sha") != kernel_source_hash():
        return None
    try:
        return int(float(vals["fetch_bytes"]) + float(vals["write_bytes"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, plans, max_segments: int, min_seconds: float = 10.0, max_passes: int = 5):
    """The oracle as it stands (plain C, one thread) on the first segments,
    repeated until about min_seconds of CPU work have been timed."""
    import numpy as np
    import oracle

    segs = list(zip(w.segments, plans))[:max_segments]
    n = sum(s.x.size for s, _ in segs)
    outs = [np.empty(oracle.max_bytes(seg.x.size), dtype=np.uint8) for seg, _ in segs]
    decs = [np.empty(seg.x.size, dtype=np.uint16) for seg, _ in segs]
    t_enc = t_dec = 0.0
    passes = 0
    while passes < max_passes and (passes == 0 or t_enc + t_dec < min_seconds):
        for (seg, plan), out, dec in zip(segs, outs, decs):
            t0 = time.perf_counter()
            total = oracle.encode_into(seg.x, plan, out)
            t1 = time.perf_counter()
            rc = oracle.decode_into(out[:total], seg.x.size, dec)
            t2 = time.perf_counter()
            if rc != 0 or not np.array_equal(dec, seg.x):
                raise RuntimeError("oracle round trip failed on the CPU sample")
            t_enc += t1 - t0
            t_dec += t2 - t1
        passes += 1
    gb = 2.0 * n * passes / 1e9
    return {"value": round(gb / (t_enc + t_dec), 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "first %d of %d segments (%d BF16 values), compress + decompress, %d pass(es), "
                      "single-threaded plain C -O2" % (len(segs), len(w.segments), n, passes),
            "compress_gbps": round(gb / t_enc, 4), "decompress_gbps": round(gb / t_dec, 4),
            "seconds": round(t_enc + t_dec, 3)}


REDUCE_WARMUP_CALLS = 150


def reduce_measurement(zc, steps: int) -> dict:
    """The receive side of a reduce-scatter run as a zipped all-to-all (section
    2.D): one rank's 32 Mi-value shard, compressed contributions of 7 peers
    plus the local share, reduced by zc_decompress_reduce.  Peer p's values are
    N(0, sigma_p^2) with sigma_p the first eight layer sigmas of the gradient
    bucket, each compressed with its own plan.  HIP events around K calls,
    after REDUCE_WARMUP_CALLS calls: per-call timings on MI355X show about 20
    fast calls, then about 80 calls some 20 % slower, then a steady state (the
    device settling after a burst of this kernel), which is what a training
    job that reduces bucket after bucket sees."""
    import numpy as np
    import torch

    from lossless_bf16_exponent_amd import workloads

    n, peers = 1 << 25, 7
    sig = workloads.config3_sigmas()[:peers + 1]
    g = np.random.default_rng(21)
    xs = [torch.from_numpy(workloads.bf16_bits_from_f32(g.standard_normal(n).astype(np.float32)
                                                          * np.float32(s)).view(np.int16)).cuda() for s in sig]
    cap = zc.zc_max_compressed_bytes(n)
    bufs = [torch.empty(cap, dtype=torch.uint8, device="cuda") for _ in range(peers)]
    sizes = torch.zeros(peers, dtype=torch.int64, device="cuda")
    for p in range(peers):
        zc.zc_compress(xs[p + 1], n, zc.zc_plan_from_sigma(float(sig[p + 1])), bufs[p], cap, sizes.data_ptr() + 8 * p)
    torch.cuda.synchronize()
    totals = [int(v) for v in sizes.cpu()]
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    ptrs = [b.data_ptr() for b in bufs]
    for _ in range(REDUCE_WARMUP_CALLS):
        zc.zc_decompress_reduce(ptrs, totals, n, xs[0], out, None, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        zc.zc_decompress_reduce(ptrs, totals, n, xs[0], out, None, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    alg = sum(totals) + 4 * n  # the peer streams and the local share read, the result written
    achieved = alg / (ms * 1e-3) / 1e9
    return {"shard_values": n, "peers": peers, "local": True, "warmup_calls": REDUCE_WARMUP_CALLS,
            "us": round(ms * 1e3, 2),
            "uncompressed_gbps": round(2.0 * n * (peers + 1) / (ms * 1e-3) / 1e9, 1),
            "algorithmic_bytes": int(alg), "achieved_gbps": round(achieved, 1),
            "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4), "kernel": "reduce_kernel"}


def stats_measurement(zc, x, seg_ns, steps: int) -> dict:
    """The online statistics that section 2.A replaces by its sigma-derived
    table, on the resident gradient bucket: the exponent histogram and the
    sigma estimate of the whole buffer (HIP events around K back-to-back
    calls; algorithmic bytes = the 2n input bytes read), and the wall time of
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
        for _ in range(3):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
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


def fallback_measurement(zc, steps: int) -> dict:
    """The raw fallback on the stress workload that coding expands most
    (2^24 uniformly random non-NaN/Inf BF16 patterns under the sigma = 0.02
    plan, 18.8 bits per value coded): compress with ZC_PLAN_RAW_FALLBACK (the
    coded pass, then the raw pass that copies the input behind the raw header)
    and decompress of the raw stream, HIP events around K calls each."""
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
    enc_call = lambda: zc.zc_compress(x, n, plan, out, cap, size, stream)
    dec_call = lambda: zc.zc_decompress(out, cap, n, dec, None, stream)
    enc_call()
    dec_call()
    torch.cuda.synchronize()
    total = int(size.item())
    if total != 128 + 2 * n or out[31].item() != 1 or not torch.equal(dec, x):
        raise RuntimeError("the fallback did not give a lossless raw stream")
    res = {"workload": w.name, "values": n, "stream_bytes": total, "raw": True}
    for name, call in (("compress", enc_call), ("decompress", dec_call)):
        for _ in range(3):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name + "_us"] = round(ms * 1e3, 2)
        res[name + "_gbps"] = round(2.0 * n / (ms * 1e-3) / 1e9, 1)
    res["kernels"] = {"compress": "compress_kernel + raw_pass_kernel", "decompress": "decode_kernel (raw branch)"}
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="3", help="workload id (1, 2, 3, 4, 5a, 5b); default 3")
    ap.add_argument("--cpu-segments", type=int, default=32, help="segments in the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reduce", action="store_true", help="skip the reduce-scatter receive-side measurement")
    ap.add_argument("--no-stats", action="store_true", help="skip the histogram / sigma-estimate measurement")
    ap.add_argument("--no-fallback", action="store_true", help="skip the raw-fallback measurement")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the codec on one GPU; runs on several GPUs are not supported "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from lossless_bf16_exponent_amd import workloads, zc

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)

    t_gen = time.perf_counter()
    w = workloads.get(args.workload)
    print("# workload %s: %d values in %d segments, generated in %.1f s"
          % (w.name, w.n, len(w.segments), time.perf_counter() - t_gen), file=sys.stderr, flush=True)

    t0 = time.perf_counter()
    plans = [zc.zc_plan_from_sigma(seg.sigma) for seg in w.segments]
    plan_us = (time.perf_counter() - t0) * 1e6 / len(plans)

    x = torch.from_numpy(w.buffer.view(np.int16)).cuda()
    ns = [seg.x.size for seg in w.segments]
    offs = np.concatenate([[0], np.cumsum(ns)]).astype(np.int64)
    caps = [zc.zc_max_compressed_bytes(n) for n in ns]
    slots = [(c + 255) // 256 * 256 for c in caps]
    soff = np.concatenate([[0], np.cumsum(slots)]).astype(np.int64)
    out = torch.empty(int(soff[-1]), dtype=torch.uint8, device="cuda")
    sizes = torch.zeros(len(ns), dtype=torch.int64, device="cuda")
    dec = torch.empty_like(x)
    status = torch.zeros(len(ns), dtype=torch.int32, device="cuda")
    xb, ob, db = x.data_ptr(), out.data_ptr(), dec.data_ptr()
    enc_segs = zc.make_enc_segs([(xb + 2 * int(offs[i]) if ns[i] else 0, ns[i], plans[i], ob + int(soff[i]),
                                  caps[i], sizes.data_ptr() + 8 * i) for i in range(len(ns))])
    dec_segs = zc.make_dec_segs([(ob + int(soff[i]), caps[i], ns[i], db + 2 * int(offs[i]) if ns[i] else 0, 0)
                                 for i in range(len(ns))])
    chk_segs = zc.make_dec_segs([(ob + int(soff[i]), caps[i], ns[i], db + 2 * int(offs[i]) if ns[i] else 0,
                                  status.data_ptr() + 4 * i) for i in range(len(ns))])
    stream = torch.cuda.current_stream()

    # correctness of what is timed: one checked round trip first
    zc.zc_compress_batch(enc_segs, stream)
    zc.zc_decompress_batch(chk_segs, stream)
    torch.cuda.synchronize()
    if status.any() or not torch.equal(dec, x):
        print("bench.py: GPU round trip is not lossless", file=sys.stderr)
        return 1
    totals = sizes.cpu().numpy()
    stream_bytes = int(totals.sum())
    zero_points = 0
    for i in range(len(ns)):
        o = int(soff[i])
        zero_points += int.from_bytes(out[o + 32:o + 40].cpu().numpy().tobytes(), "little")

    n = w.n
    for _ in range(args.warmup):
        zc.zc_compress_batch(enc_segs, stream)
        zc.zc_decompress_batch(dec_segs, stream)
    torch.cuda.synchronize()

    # timed region 1, the whole hot path: K steps of one batched compress and
    # one batched decompress, with nothing recorded between the launches
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    g0.record(stream)
    for _ in range(args.steps):
        zc.zc_compress_batch(enc_segs, stream)
        zc.zc_decompress_batch(dec_segs, stream)
    g1.record(stream)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    gpu_step_ms = g0.elapsed_time(g1) / args.steps

    # timed region 2, per call: HIP events on the launch stream around K
    # back-to-back compress calls, then K back-to-back decompress calls
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    for _ in range(args.steps):
        zc.zc_compress_batch(enc_segs, stream)
    e[1].record(stream)
    for _ in range(args.steps):
        zc.zc_decompress_batch(dec_segs, stream)
    e[2].record(stream)
    torch.cuda.synchronize()
    enc_ms = e[0].elapsed_time(e[1]) / args.steps
    dec_ms = e[1].elapsed_time(e[2]) / args.steps
    if not torch.equal(dec, x):
        print("bench.py: decoded buffer differs after timing", file=sys.stderr)
        return 1

    # practical ceiling: a device-to-device copy of the input
    cp = torch.empty_like(x)
    for _ in range(3):
        cp.copy_(x)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        cp.copy_(x)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / 10
    del cp

    ms_per_step = t_total * 1e3 / args.steps
    gb = 2.0 * n / 1e9
    enc_alg = 2.0 * n + stream_bytes
    dec_alg = stream_bytes + 2.0 * n
    calls = {"compress": (enc_ms, enc_alg, "compress_kernel"),
             "decompress": (dec_ms, dec_alg, "decode_kernel")}
    dom = max(calls, key=lambda k: calls[k][0])
    dom_ms, dom_bytes, dom_kernels = calls[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
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
        "config": {"workload": w.name, "values": n, "segments": len(ns), "input": "bf16",
                   "description": w.description, "launches_per_step": "1 batched compress + 1 batched decompress"},
        "compress_gbps": round(gb / (enc_ms * 1e-3), 2),
        "decompress_gbps": round(gb / (dec_ms * 1e-3), 2),
        "compress_us": round(enc_ms * 1e3, 2),
        "decompress_us": round(dec_ms * 1e3, 2),
        "compress_hbm_frac": round(enc_alg / (enc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "decompress_hbm_frac": round(dec_alg / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "compression_ratio": round(stream_bytes / (2.0 * n), 5),
        "bits_per_value": round(8.0 * stream_bytes / n, 4),
        "zero_point_rate": round(zero_points / n, 6),
        "copy_ceiling_gbps": round(4.0 * n / (copy_ms * 1e-3) / 1e9, 1),
        "plan_us": round(plan_us, 2),
        "device": dev_name,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "call": dom, "kernels": dom_kernels, "algorithmic_bytes": int(dom_bytes),
                     "avg_launch_us": round(dom_ms * 1e3, 2)},
        "gpu_step_ms": round(gpu_step_ms, 4),
        "kernel_sha": kernel_source_hash(),
    }
    if not args.no_stats:
        rec["plan_variants"] = stats_measurement(zc, x, ns, args.steps)
        rec["plan_variants"]["sigma_table_us_per_bucket"] = round(plan_us * len(ns), 2)
    if not args.no_reduce or not args.no_fallback:
        del out, dec
        torch.cuda.empty_cache()
    if not args.no_fallback:
        rec["raw_fallback"] = fallback_measurement(zc, args.steps)
    if not args.no_reduce:
        rec["reduce_scatter_local"] = reduce_measurement(zc, args.steps)
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, plans, args.cpu_segments)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
