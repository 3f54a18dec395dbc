#!/usr/bin/env python3
"""KV-cache GB/s read by the fused 4-bit attend, on one MI355X.

One step = one ``kvq_attend`` call (the fused path: K/V tile loads, in-register
decode, scores, online softmax (m, z, u), split combine) over one full
synthetic packed cache of the chosen workload, with Q, the packed cache, the
output and the workspace resident in HBM before timing starts.  Packing is
outside the step, as in the pages' timing scope; it, the decode-all
baseline (kvq_dequant + kvq_attend_f32) and a plain streaming read of the
same byte count (kvq_stream_read, the measured HBM ceiling) are timed
separately and reported under "extra".

The timed steps rotate over enough distinct copies of the packed cache that
their total exceeds the 256 MB Infinity Cache, so every step streams its KV
bytes from HBM.  By default they are replayed from a HIP graph holding one
step per cache copy (captured once, checked bit for bit against the eager
result before timing), so that a ~13 us kernel is not paced by the host's
per-call launch cost; `--launch eager` times a plain Python loop of calls.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import WORKLOADS, make_qkv  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MALL_BYTES = 256 * 2 ** 20     # Infinity Cache
METRIC = "KV-cache GB/s read by fused 4-bit attend (and % of HBM peak) at n=4096, GQA 32/8"


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def kv_bytes(w, bits, group):
    """Algorithmic bytes one attend reads: every K and V code byte and float32
    scale once (2 * B * Hkv * N * D * (bits/8 + 4/group))."""
    npad = -(-w.N // group) * group
    dpad = -(-w.D // group) * group
    per_head = (w.D * npad + w.N * dpad) * bits // 8 + 4 * (w.D * npad // group + w.N * dpad // group)
    return w.B * w.Hkv * per_head


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attend_mfma_gqa_n4096_traffic.md")
# The sources the measured kernel is compiled from (its file, the shared header
# and the build script with its flags).
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_kv_cache_attend_amd", "csrc", f)
                  for f in ("kvq_attend_mfma.hip", "kvq_mfma_common.h", "kvq_internal.h")] + [
                      os.path.join(ROOT, "quantized_kv_cache_attend_amd", "build.py")]


def kernel_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def dtype_label(bits, group, variant):
    """What the timed kernel computes in: the matrix-core kernels (group 32)
    take exact fp16 code operands and fp16 hi + lo float32 factors; the
    streaming and general kernels decode to float32."""
    if variant in ("auto", "mfma") and group == 32:
        return f"u{bits} codes + f32 scales; fp16 hi+lo matrix-core operands, f32 accumulate"
    return f"u{bits} codes + f32 scales; f32 decode and arithmetic"


def measured_traffic():
    """HBM bytes per launch of the matrix-core attend kernel from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by the same
    counter's reading for a copy of known size), or None when the summary is
    missing or was taken on a different kernel source (sha256 over
    KERNEL_SOURCES)."""
    try:
        text = open(TRAFFIC_FILE, encoding="utf-8").read()
        src = kernel_source_sha256()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch:", "kernel_source_sha256:")))
    if fields.get("kernel_source_sha256", "").strip() != src:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


def copy_calibration(mib, reps):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = mib * 2 ** 20 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {mib} MiB (read {mib} MiB, write {mib} MiB each)")


def cpu_baseline(w, q, k, v, bits, group, seconds):
    """Time the float64 oracle (decode the whole packed cache, dense attention)
    on this host, as it stands, over whole passes of the workload until
    `seconds` have elapsed (at least 2 passes)."""
    from oracle import kvq_oracle as O
    kc, ks = O.pack_k(k, bits, group)
    vc, vs = O.pack_v(v, bits, group)
    times = []
    t_start = time.perf_counter()
    while len(times) < 2 or time.perf_counter() - t_start < seconds:
        t0 = time.perf_counter()
        O.attend_packed(q, kc, ks, vc, vs, w.N, bits, group)
        times.append(time.perf_counter() - t0)
    threads = None
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info())
    except Exception:
        pass
    cores = len(os.sched_getaffinity(0))
    med = float(np.median(times))
    return {
        "value": kv_bytes(w, bits, group) / med / 1e9,
        "unit": "GB/s",
        "cores": int(threads or cores),
        "kind": "oracle",
        "sample": (f"{len(times)} full passes of {w.name} (decode all {w.B * w.Hkv} KV heads to "
                   f"float32, dense float64 attention), median {med * 1e3:.1f} ms/pass; "
                   f"{cores} host cores visible, BLAS threads {threads}"),
    }


def long_context_line(launch, sink):
    """The long-context workload (batch 16, 32768 tokens, GQA 64/8, 4 queries
    per head: 32 query rows per KV head, the 32-row matrix-core kernel) at its
    16 KV splits: per-call time of the fused attend over rotating cache copies
    past the Infinity Cache, launched like the main step, beside a streaming
    read of the same byte count."""
    import torch
    import quantized_kv_cache_attend_amd as kvq
    w = WORKLOADS["gqa_n32768"]
    bits, group = w.formats[0]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    q, k, v = make_qkv(w, 0)
    qd = torch.from_numpy(q).to(dev)
    kd = torch.from_numpy(k).to(dev)
    del k
    kc, ks = kvq.pack_k(kd, bits, group)
    del kd
    vd = torch.from_numpy(v).to(dev)
    del v
    vc, vs = kvq.pack_v(vd, bits, group)
    del vd
    nbytes = kv_bytes(w, bits, group)
    copies = max(2, math.ceil(3 * MALL_BYTES / nbytes))
    caches = [(kc, ks, vc, vs)] + [tuple(t.clone() for t in (kc, ks, vc, vs))
                                   for _ in range(copies - 1)]
    out = torch.empty_like(qd)
    ws = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D, w.num_splits, device=dev)

    def one_pass():
        for c in caches:
            kvq.attend(qd, *c, w.N, bits, group, num_splits=w.num_splits, workspace=ws, out=out)
    one_pass()
    torch.cuda.synchronize()
    ref = out.clone()
    run = one_pass
    if launch == "graph":
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            one_pass()
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError("gqa_n32768 graph replay differs from the eager result")
        run = g.replay

    def timed_passes(fn, n):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    n_pass = max(2, 400 // copies)
    us = timed_passes(run, n_pass) / copies
    if not torch.equal(out, ref):
        raise RuntimeError("gqa_n32768 timed calls changed the output")
    del caches, kc, ks, vc, vs

    rbytes = (nbytes + 15) // 16 * 16
    bufs = [torch.zeros(rbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]

    def reads():
        for b in bufs:
            kvq.stream_read(b, sink)
    read_run = reads
    if launch == "graph":
        rg = torch.cuda.CUDAGraph()
        reads()
        torch.cuda.synchronize()
        with torch.cuda.graph(rg):
            reads()
        read_run = rg.replay
    read_us = timed_passes(read_run, n_pass) / copies
    del bufs
    gbs = nbytes / (us * 1e-6) / 1e9
    line = {"splits": w.num_splits, "us": round(us, 2), "kv_bytes": nbytes,
            "kv_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "read_ceiling_us": round(read_us, 2),
            "attend_over_read_ceiling": round(us / read_us, 3),
            "cache_copies": copies, "kernel": "32-row matrix-core"}
    log(f"[bench] gqa_n32768 at {w.num_splits} splits: {us:.1f} us ({gbs:.0f} GB/s, "
        f"{gbs / HBM_PEAK_GBS:.1%} of peak); streaming read {read_us:.1f} us")
    return line


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="timed steps replayed from a HIP graph (one step per cache copy) "
                         "or launched one by one from Python")
    ap.add_argument("--workload", default="gqa_n4096", choices=["gqa_n4096", "gqa_n32768"])
    ap.add_argument("--variant", default="auto", choices=["auto", "valu", "mfma", "stream"])
    ap.add_argument("--splits", type=int, default=-1, help="-1: workload default, 0: auto")
    ap.add_argument("--bits", type=int, default=0, choices=[0, 4, 8],
                    help="code width of the timed cache (0: the workload's, 4)")
    ap.add_argument("--group", type=int, default=0, help="group length (0: the workload's, 32)")
    ap.add_argument("--copies", type=int, default=0, help="cache copies to rotate (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip pack / decode-all timings")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run device copies of MIB MiB (for counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention shards by (batch, KV head) with no exchange; one GPU shows its share)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, 5)
        return

    import torch
    import quantized_kv_cache_attend_amd as kvq

    w = WORKLOADS[args.workload]
    bits, group = w.formats[0]
    default_format = not args.bits and not args.group
    bits, group = args.bits or bits, args.group or group
    splits = w.num_splits if args.splits < 0 else args.splits
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log(f"[bench] workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} R={w.R} N={w.N} D={w.D} "
        f"{bits}-bit g{group} splits={splits or 'auto'}")
    q, k, v = make_qkv(w, 0)
    qd, kd, vd = (torch.from_numpy(a).to(dev) for a in (q, k, v))
    kc, ks = kvq.pack_k(kd, bits, group)
    vc, vs = kvq.pack_v(vd, bits, group)
    torch.cuda.synchronize()
    nbytes = kv_bytes(w, bits, group)
    assert nbytes == kc.numel() + vc.numel() + 4 * (ks.numel() + vs.numel())

    copies = args.copies or max(2, math.ceil(3 * MALL_BYTES / nbytes))
    caches = [(kc, ks, vc, vs)] + [tuple(t.clone() for t in (kc, ks, vc, vs)) for _ in range(copies - 1)]
    out = torch.empty_like(qd)
    ws = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D, splits, device=dev)
    stream = torch.cuda.current_stream(dev)
    log(f"[bench] {copies} cache copies x {nbytes / 1e6:.1f} MB = {copies * nbytes / 1e6:.0f} MB")

    def step(i):
        c = caches[i % copies]
        kvq.attend(qd, *c, w.N, bits, group, num_splits=splits, workspace=ws, out=out,
                   variant=args.variant)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ref = out.clone()      # every cache copy holds the same bytes: one expected output

    def eager_steps(n):
        for i in range(n):
            step(i)

    run_steps = eager_steps
    if args.launch == "graph":
        # One graph node per cache copy, on torch's capture stream (default
        # priority); the kernel resets its own split counters, so replays need
        # no memset nodes.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_steps(copies)
        torch.cuda.synchronize()
        for rep in range(3):     # replays checked bit for bit, eager work between them
            out.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, ref):
                raise RuntimeError(f"graph replay {rep} differs from the eager result")
            eager_steps(1)
            torch.cuda.synchronize()

        def run_steps(n):
            for _ in range(n // copies):
                graph.replay()
            eager_steps(n % copies)
        run_steps(args.warmup)
        torch.cuda.synchronize()

    # Timed region: K steps back to back, host clock and stream events.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    run_steps(args.steps)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    region_ms = e0.elapsed_time(e1) / args.steps
    if not torch.equal(out, ref):
        raise RuntimeError("timed steps changed the output")
    log(f"[bench] {args.launch}: wall {ms_per_step * 1e3:.2f} us/step, "
        f"stream events {region_ms * 1e3:.2f} us/step")

    eager_us = None
    if args.launch == "graph":
        # For comparison: the same steps launched one by one from Python.
        n_e = min(args.steps, 2000)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        eager_steps(n_e)
        torch.cuda.synchronize()
        eager_us = (time.perf_counter() - t1) * 1e6 / n_e
        log(f"[bench] eager Python loop: {eager_us:.2f} us/step")

    # Per-launch duration: an event pair around each call (same stream).
    n_ev = min(args.steps, 400)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for i in range(n_ev):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]) * 1e3  # us
    launch_us = float(np.median(per_launch))
    log(f"[bench] per-launch events: median {launch_us:.2f} us, mean {per_launch.mean():.2f}, "
        f"min {per_launch.min():.2f}, max {per_launch.max():.2f}")

    kernel_us = min(launch_us, region_ms * 1e3)
    achieved = nbytes / (kernel_us * 1e-6) / 1e9
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    finite = bool(torch.isfinite(out).all().item())

    extra = {"wall_us_per_step": round(ms_per_step * 1e3, 3),
             "stream_event_us_per_step": round(region_ms * 1e3, 3),
             "per_launch_event_us_median": round(launch_us, 3),
             "launch": (f"HIP graph of {copies} steps, replayed" if args.launch == "graph"
                        else "eager Python loop"),
             "eager_wall_us_per_step": None if eager_us is None else round(eager_us, 3),
             "cache_copies": copies, "splits": splits or "auto",
             "variant": args.variant, "output_finite": finite}

    if not args.no_extra:
        # Pack (outside the step) and the decode-all baseline, same protocol.
        kf = torch.empty_like(kd)
        vf = torch.empty_like(vd)

        def timed(fn, reps):
            fn()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / reps

        reps = 20 if w.N <= 4096 else 3
        pack_us = timed(lambda: (kvq.pack_k(kd, bits, group), kvq.pack_v(vd, bits, group)), reps)

        def decode_all():
            kvq.dequant_k(kc, ks, w.N, w.D, bits, group, out=kf)
            kvq.dequant_v(vc, vs, w.N, w.D, bits, group, out=vf)
            kvq.attend_f32(qd, kf, vf, num_splits=splits, workspace=ws, out=out)
        dec_us = timed(decode_all, reps)

        def dequant_only():
            kvq.dequant_k(kc, ks, w.N, w.D, bits, group, out=kf)
            kvq.dequant_v(vc, vs, w.N, w.D, bits, group, out=vf)
        deq_us = timed(dequant_only, reps)
        # HBM bytes of decode-all: read the packed cache, write and read back
        # the float32 K and V.
        f32_bytes = 2 * kd.numel() * 4
        extra.update({"pack_us": round(pack_us, 1), "decode_all_us": round(dec_us, 1),
                      "decode_all_dequant_us": round(deq_us, 1),
                      "decode_all_kv_gbs": round(nbytes / (dec_us * 1e-6) / 1e9, 1),
                      "decode_all_hbm_bytes": nbytes + 2 * f32_bytes})
        log(f"[bench] pack {pack_us:.1f} us, decode-all baseline {dec_us:.1f} us "
            f"(dequant {deq_us:.1f} us + float32 attend {dec_us - deq_us:.1f} us)")

        # Measured ceiling: a plain streaming read (kvq_stream_read) of the
        # same byte count, rotating over as many buffers as the cache copies.
        rbytes = (nbytes + 15) // 16 * 16
        bufs = [torch.zeros(rbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        def reads():
            for b in bufs:
                kvq.stream_read(b, sink)
        reads()
        torch.cuda.synchronize()
        read_pass = reads
        if args.launch == "graph":      # launched the same way as the timed steps
            rgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(rgraph):
                reads()
            read_pass = rgraph.replay
        n_pass = max(1, min(args.steps, 2000) // copies)
        read_pass()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n_pass):
            read_pass()
        b_.record(stream)
        torch.cuda.synchronize()
        read_us = a.elapsed_time(b_) * 1e3 / (n_pass * copies)
        del bufs
        extra.update({"read_ceiling_us": round(read_us, 3),
                      "read_ceiling_gbs": round(rbytes / (read_us * 1e-6) / 1e9, 1),
                      "attend_over_read_ceiling": round(kernel_us / read_us, 3)})
        log(f"[bench] streaming-read ceiling for the same bytes: {read_us:.2f} us "
            f"({rbytes / (read_us * 1e-6) / 1e9:.0f} GB/s); attend / ceiling = {kernel_us / read_us:.2f}")

        # Decode loop on a growing cache laid out for all N tokens: a prompt
        # of N - 80 tokens in one append, then one-token steps over the
        # tokens so far, 16 untimed and 64 timed with one event pair around
        # the 64 (eager: each step's N differs).  Two forms of the step: one
        # kvq_append_attend call (one launch where the 4-row matrix-core
        # kernel serves it), and kvq_append followed by kvq_attend_cache.  The
        # last step attends all N tokens and must equal the full-cache call
        # above bit for bit.
        n_warm, n_timed = 16, 64
        prompt = w.N - n_warm - n_timed
        if prompt >= 1:
            kp, vp = kd[:, :, :prompt].contiguous(), vd[:, :, :prompt].contiguous()
            cache = kvq.new_cache(w.B, w.Hkv, w.N, w.D, bits, group, device=dev)
            cache2 = kvq.new_cache(w.B, w.Hkv, w.N, w.D, bits, group, device=dev)
            p0 = torch.cuda.Event(enable_timing=True)
            p1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            p0.record(stream)
            kvq.append(kp, vp, 0, cache, w.N, bits, group)
            p1.record(stream)
            kvq.append(kp, vp, 0, cache2, w.N, bits, group)
            torch.cuda.synchronize()
            prompt_us = p0.elapsed_time(p1) * 1e3
            del kp, vp
            k_steps = [kd[:, :, i:i + 1].contiguous() for i in range(prompt, w.N)]
            v_steps = [vd[:, :, i:i + 1].contiguous() for i in range(prompt, w.N)]
            dec_out = torch.empty_like(qd)
            dec_out2 = torch.empty_like(qd)
            ws2 = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D, splits, device=dev)
            torch.cuda.synchronize()
            # Queue each loop behind a few ms of unrelated reads so the host
            # enqueues every step before the GPU reaches them: one event pair
            # then times back-to-back GPU work, not the pace of the Python
            # calls (an event pair around one small kernel costs several us).
            blocker = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)

            def queue_blocker():
                for _ in range(128):
                    kvq.stream_read(blocker, sink)
            d0 = torch.cuda.Event(enable_timing=True)
            d1 = torch.cuda.Event(enable_timing=True)
            queue_blocker()
            for i, n in enumerate(range(prompt, w.N)):
                if i == n_warm:
                    d0.record(stream)
                kvq.append_attend(qd, k_steps[i], v_steps[i], n, cache2, w.N, bits, group,
                                  num_splits=splits, workspace=ws2, out=dec_out2)
            d1.record(stream)
            torch.cuda.synchronize()
            fused_us = d0.elapsed_time(d1) * 1e3 / n_timed
            queue_blocker()
            for i, n in enumerate(range(prompt, w.N)):
                if i == n_warm:
                    d0.record(stream)
                kvq.append(k_steps[i], v_steps[i], n, cache, w.N, bits, group)
                kvq.attend(qd, *cache[:4], n + 1, bits, group, num_splits=splits, workspace=ws,
                           out=dec_out, variant=args.variant, capacity=w.N)
            d1.record(stream)
            torch.cuda.synchronize()
            step_us = d0.elapsed_time(d1) * 1e3 / n_timed
            full = kvq.attend(qd, kc, ks, vc, vs, w.N, bits, group, num_splits=splits,
                              workspace=ws, variant=args.variant)
            torch.cuda.synchronize()
            same = bool(torch.equal(dec_out, full))
            same_fused = bool(torch.equal(dec_out2, full)) and all(
                torch.equal(a, b) for a, b in zip(cache, cache2))
            # the same number of back-to-back attends alone (all N tokens)
            queue_blocker()
            d0.record(stream)
            for _ in range(n_timed):
                kvq.attend(qd, *cache[:4], w.N, bits, group, num_splits=splits, workspace=ws,
                           out=dec_out, variant=args.variant, capacity=w.N)
            d1.record(stream)
            torch.cuda.synchronize()
            attend_us = d0.elapsed_time(d1) * 1e3 / n_timed
            extra["decode_step"] = {
                "tokens": f"{w.N - n_timed + 1}..{w.N}",
                "prompt_append_us": round(prompt_us, 1),
                "prompt_tokens": prompt,
                "step_us": round(fused_us, 3),
                "step_form": "kvq_append_attend (append in the attend's launch)",
                "attend_only_us": round(attend_us, 3),
                "append_us": round(fused_us - attend_us, 3),
                "two_call_step_us": round(step_us, 3),
                "two_call_append_us": round(step_us - attend_us, 3),
                "last_step_equals_full_cache_attend": same and same_fused,
            }
            log(f"[bench] decode steps: {fused_us:.2f} us per one-call append + attend, "
                f"{step_us:.2f} us as two calls, attend alone {attend_us:.2f} us (back to back, "
                f"{n_timed} steps); last step == full-cache attend: {same and same_fused}")
            del cache, cache2, blocker, ws2

        # A causal multi-token step on the same cache: R_c = 4 new queries per
        # head (the last 4 positions; GQA makes 4 * Hq/Hkv rows per KV head),
        # against the same queries without the mask.  Events around 200
        # calls rotating over the cache copies, enqueued behind a blocker.
        r_c = 4
        qc = torch.from_numpy(make_qkv(dataclasses.replace(w, R=r_c), 1, n=1)[0]).to(dev)
        out_c = torch.empty_like(qc)
        ws_c = kvq.new_workspace(w.B, w.Hq, w.Hkv, r_c, w.N, w.D, 0, device=dev)
        timings = {}
        for causal in (True, False):
            kvq.attend(qc, *caches[0], w.N, bits, group, workspace=ws_c, out=out_c,
                       causal=causal)
            torch.cuda.synchronize()
            blocker = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
            for _ in range(64):
                kvq.stream_read(blocker, sink)
            c0 = torch.cuda.Event(enable_timing=True)
            c1 = torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            for i in range(200):
                kvq.attend(qc, *caches[i % copies], w.N, bits, group, workspace=ws_c, out=out_c,
                           causal=causal)
            c1.record(stream)
            torch.cuda.synchronize()
            timings[causal] = c0.elapsed_time(c1) * 1e3 / 200
            del blocker
        extra["causal_step"] = {
            "queries_per_head": r_c, "rows_per_kv_head": r_c * w.Hq // w.Hkv,
            "causal_us": round(timings[True], 3), "unmasked_us": round(timings[False], 3),
            "causal_kv_gbs": round(nbytes / (timings[True] * 1e-6) / 1e9, 1),
        }
        log(f"[bench] causal step of {r_c} queries per head: {timings[True]:.2f} us "
            f"(unmasked {timings[False]:.2f} us)")

        # The mixed cache: the 64 most recent tokens in float32, the rest
        # packed (kvq_attend_window: window parts in the matrix-core launch),
        # same queries.
        win = 64
        kpre = kvq.pack_k(kd[:, :, :w.N - win].contiguous(), bits, group)
        vpre = kvq.pack_v(vd[:, :, :w.N - win].contiguous(), bits, group)
        kw, vw = kd[:, :, w.N - win:].contiguous(), vd[:, :, w.N - win:].contiguous()
        out_w = torch.empty_like(qd)
        ws_w = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D,
                                 (splits or kvq.auto_splits(w.B, w.Hkv, w.N)) + win // 32,
                                 device=dev)

        def window_call():  # a workspace slot per 32 window tokens beyond the splits: fused form
            kvq.attend_window(qd, *kpre, *vpre, kw, vw, w.N - win, bits, group, workspace=ws_w,
                              out=out_w, num_splits=splits)
        window_call()
        torch.cuda.synchronize()
        blocker = torch.empty(256 * 2 ** 20, dtype=torch.uint8, device=dev)
        for _ in range(64):
            kvq.stream_read(blocker, sink)
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        n_w = 20
        w0.record(stream)
        for _ in range(n_w):
            window_call()
        w1.record(stream)
        torch.cuda.synchronize()
        win_us = w0.elapsed_time(w1) * 1e3 / n_w
        extra["window_step"] = {"float32_window_tokens": win, "us": round(win_us, 2),
                                "form": "one matrix-core launch: packed splits, then window "
                                        "parts, merged in its split combine"}
        log(f"[bench] mixed cache (last {win} tokens float32): {win_us:.1f} us")
        del blocker, kpre, vpre, kw, vw, ws_w

        # The other formats on the same cache shape: 8-bit group 32 (the
        # matrix-core kernels), 4-bit and 8-bit group 8 (the streaming kernel)
        # and 4-bit group 8 on the general kernel, KV GB/s of their own byte
        # counts, timed like the main step (rotating cache copies past the
        # Infinity Cache, launched the same way).
        fmt = {}
        for fb, fg, fvar in ((8, 32, "auto"), (4, 8, "auto"), (8, 8, "auto"), (4, 8, "valu")):
            fbytes = kv_bytes(w, fb, fg)
            fcopies = max(2, math.ceil(3 * MALL_BYTES / fbytes))
            fk0, fks0 = kvq.pack_k(kd, fb, fg)
            fv0, fvs0 = kvq.pack_v(vd, fb, fg)
            fcaches = [(fk0, fks0, fv0, fvs0)] + [tuple(t.clone() for t in (fk0, fks0, fv0, fvs0))
                                                  for _ in range(fcopies - 1)]
            fout = torch.empty_like(qd)

            def fpass():
                for c in fcaches:
                    kvq.attend(qd, *c, w.N, fb, fg, workspace=ws, out=fout, num_splits=splits,
                               variant=fvar)
            fpass()
            torch.cuda.synchronize()
            fref = fout.clone()
            run_f = fpass
            if args.launch == "graph":
                fgraph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(fgraph):
                    fpass()
                torch.cuda.synchronize()
                fout.fill_(float("nan"))
                fgraph.replay()
                torch.cuda.synchronize()
                if not torch.equal(fout, fref):
                    raise RuntimeError(f"{fb}-bit g{fg} graph replay differs from the eager result")
                run_f = fgraph.replay
            n_f = max(2, 400 // fcopies)
            f0 = torch.cuda.Event(enable_timing=True)
            f1 = torch.cuda.Event(enable_timing=True)
            f0.record(stream)
            for _ in range(n_f):
                run_f()
            f1.record(stream)
            torch.cuda.synchronize()
            fus = f0.elapsed_time(f1) * 1e3 / (n_f * fcopies)
            key = f"{fb}bit_g{fg}" + ("_general_kernel" if fvar == "valu" else "")
            fmt[key] = {"us": round(fus, 2), "kv_bytes": fbytes,
                        "kv_gbs": round(fbytes / (fus * 1e-6) / 1e9, 1),
                        "hbm_frac": round(fbytes / (fus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "kernel": ("general" if fvar == "valu" else
                                   "matrix-core" if fg == 32 else "streaming"),
                        "cache_copies": fcopies}
            del fcaches, fk0, fks0, fv0, fvs0, fout
            if args.launch == "graph":
                del fgraph
        extra["other_formats"] = fmt
        log("[bench] other formats: " +
            ", ".join(f"{k} ({v['kernel']}) {v['us']:.1f} us ({v['kv_gbs']:.0f} GB/s)"
                      for k, v in fmt.items()))

        # The streaming kernel's causal and mixed-cache forms on the same cache
        # shape in 4-bit group 8: a causal chunk of 2 queries per head (8 rows
        # per KV head) over the whole cache, and the 64 most recent tokens kept
        # in float32 with the 1-query step; rotating cache copies past the
        # Infinity Cache, timed with stream events over back-to-back calls.
        sbits, sgroup, swin = 4, 8, 64
        sbytes = kv_bytes(w, sbits, sgroup)
        scopies = max(2, math.ceil(3 * MALL_BYTES / sbytes))
        sk0 = kvq.pack_k(kd, sbits, sgroup) + kvq.pack_v(vd, sbits, sgroup)
        scaches = [sk0] + [tuple(t.clone() for t in sk0) for _ in range(scopies - 1)]
        q2 = torch.from_numpy(make_qkv(dataclasses.replace(w, R=2), 1, n=1)[0]).to(dev)
        ws2 = kvq.new_workspace(w.B, w.Hq, w.Hkv, 2, w.N, w.D, 0, device=dev)
        out2 = torch.empty_like(q2)
        wk0 = (kvq.pack_k(kd[:, :, :w.N - swin].contiguous(), sbits, sgroup) +
               kvq.pack_v(vd[:, :, :w.N - swin].contiguous(), sbits, sgroup))
        wcaches = [wk0] + [tuple(t.clone() for t in wk0) for _ in range(scopies - 1)]
        kwin, vwin = kd[:, :, w.N - swin:].contiguous(), vd[:, :, w.N - swin:].contiguous()
        ws_sw = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D,
                                  kvq.auto_splits(w.B, w.Hkv, w.N) + swin // 32, device=dev)
        outw = torch.empty_like(qd)

        def causal8(c):
            kvq.attend(q2, *c, w.N, sbits, sgroup, workspace=ws2, out=out2, causal=True)

        def window8(c):
            kvq.attend_window(qd, *c, kwin, vwin, w.N - swin, sbits, sgroup, workspace=ws_sw,
                              out=outw)

        sforms = {}
        for name, fn, cs in (("4bit_g8_causal_2_queries", causal8, scaches),
                             ("4bit_g8_window_64", window8, wcaches)):
            for c in cs[:2]:
                fn(c)
            torch.cuda.synchronize()
            n_s = max(2, 200 // len(cs))
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for _ in range(n_s):
                for c in cs:
                    fn(c)
            s1.record(stream)
            torch.cuda.synchronize()
            sforms[name] = {"us": round(s0.elapsed_time(s1) * 1e3 / (n_s * len(cs)), 2),
                            "kernel": "streaming", "cache_copies": len(cs)}
        if not (torch.isfinite(out2).all() and torch.isfinite(outw).all()):
            raise RuntimeError("streaming-kernel forms gave non-finite outputs")
        extra["streaming_forms"] = sforms
        log("[bench] streaming kernel, 4-bit g8: " +
            ", ".join(f"{k} {v['us']:.1f} us" for k, v in sforms.items()))
        del scaches, wcaches, sk0, wk0, q2, out2, outw, ws2, ws_sw

        # The single-head workloads (128 / 512 / 1024 tokens, D = 32, every
        # format they name): per-call time of one fused attend, graph-launched
        # back to back.  These are latency-bound (a few KB of cache).
        small = {}
        for sname in ("single_n128", "single_n512", "single_n1024"):
            sw = WORKLOADS[sname]
            sq, sk_, sv_ = make_qkv(sw, 0)
            sqd, skd, svd = (torch.from_numpy(a).to(dev) for a in (sq, sk_, sv_))
            for sb, sg in sw.formats:
                sc = kvq.pack_k(skd, sb, sg) + kvq.pack_v(svd, sb, sg)
                sws = kvq.new_workspace(sw.B, sw.Hq, sw.Hkv, sw.R, sw.N, sw.D, 0, device=dev)
                sout = torch.empty_like(sqd)

                def scalls(n):
                    for _ in range(n):
                        kvq.attend(sqd, *sc, sw.N, sb, sg, workspace=sws, out=sout)
                scalls(1)
                torch.cuda.synchronize()
                n_s, reps_s = 50, 10
                srun = lambda: scalls(n_s)  # noqa: E731
                if args.launch == "graph":
                    sgraph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(sgraph):
                        scalls(n_s)
                    srun = sgraph.replay
                srun()
                torch.cuda.synchronize()
                s0 = torch.cuda.Event(enable_timing=True)
                s1 = torch.cuda.Event(enable_timing=True)
                s0.record(stream)
                for _ in range(reps_s):
                    srun()
                s1.record(stream)
                torch.cuda.synchronize()
                small[f"{sname}_{sb}bit_g{sg}"] = round(s0.elapsed_time(s1) * 1e3 / (n_s * reps_s), 2)
        extra["single_head_us_per_call"] = small
        log("[bench] single-head workloads (us per call): " +
            ", ".join(f"{k} {v:.2f}" for k, v in small.items()))

        if w.name != "gqa_n32768":
            extra["gqa_n32768"] = long_context_line(args.launch, sink)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 oracle on the host ...")
        cpu = cpu_baseline(w, q, k, v, bits, group, args.cpu_seconds)
        log(f"[bench] oracle {cpu['value']:.3f} GB/s ({cpu['sample']})")

    traffic = (measured_traffic() if args.variant in ("auto", "mfma") and w.name == "gqa_n4096"
               and default_format else None)
    result = {
        "metric": METRIC if default_format else METRIC.replace("4-bit", f"{bits}-bit g{group}"),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label(bits, group, args.variant),
        "data": "synthetic (seeded N(0,1) float32 Q/K/V, packed on the GPU)",
        "config": {"workload": w.name, "batch": w.B, "n_tokens": w.N, "hq": w.Hq, "hkv": w.Hkv,
                   "queries_per_head": w.R, "head_dim": w.D, "bits": bits, "group": group,
                   "kv_bytes": nbytes, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
