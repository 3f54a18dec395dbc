"""Phase timeline of the fused attend kernels (a measurement aid).

Build the diagnostic library first (the same kernels, with per-wave phase
timestamps; see kvq_phase_trace_fetch in include/kvq.h):

    python quantized_kv_cache_attend_amd/build.py --phase-trace
    python -m quantized_kv_cache_attend_amd.phase_trace --workload gqa_n4096
    python -m quantized_kv_cache_attend_amd.phase_trace --format 4,8 --splits 8

The workload's own format (group 32) runs a matrix-core kernel; another
group (--format bits,group) runs the streaming kernel.

The workload's synthetic cache is packed with the library and copied until the
copies exceed the Infinity Cache, as in bench.py.  The diagnostic library's
kvq_attend then runs back to back over the copies, and after each batch the
records of its last launch are read.  The report gives, per phase mark, the
time since the launch's first wave started (percentiles over every recorded
wave of every batch) and each step's duration per wave (mark minus the
previous mark).  The clock is the chip-wide 100 MHz counter, so the marks of
different waves compare directly.
"""
from __future__ import annotations

import argparse
import ctypes
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import quantized_kv_cache_attend_amd as kvq  # noqa: E402
from workloads import WORKLOADS, make_qkv  # noqa: E402

LIB_PHASE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq_phase.so")
PHASE_WAVES, PHASE_MARKS = 16384, 8
MARKS = ["start", "query ready", "first block ready", "last block done", "workgroup merged",
         "partials acknowledged", "ticket taken", "end"]
MALL_BYTES = 256 * 2 ** 20


def load_phase_lib():
    if not os.path.exists(LIB_PHASE):
        raise FileNotFoundError(f"{LIB_PHASE} is missing: run build.py --phase-trace first")
    lib = ctypes.CDLL(LIB_PHASE)
    lib.kvq_attend.restype = ctypes.c_int
    lib.kvq_attend.argtypes = kvq.lib.kvq_attend.argtypes
    lib.kvq_phase_trace_fetch.restype = ctypes.c_int
    lib.kvq_phase_trace_fetch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t]
    return lib


KERNELS = {0: "4-row", 1: "32-row", 2: "streaming"}


def run(workload: str, splits: int, batches: int, per_batch: int, fmt=None):
    import torch
    w = WORKLOADS[workload]
    bits, group = fmt if fmt else w.formats[0]
    rows = w.Hq // w.Hkv * w.R
    if group == 32:
        kernel = 0 if rows <= 4 else 1
    else:
        kernel = 2
    splits = w.num_splits if splits < 0 else splits
    lib = load_phase_lib()
    q, k, v = make_qkv(w, 0)
    qd = torch.from_numpy(q).cuda()
    kc, ks = kvq.pack_k(torch.from_numpy(k).cuda(), bits, group)
    del k
    vc, vs = kvq.pack_v(torch.from_numpy(v).cuda(), bits, group)
    del v
    nbytes = kc.numel() + vc.numel() + 4 * (ks.numel() + vs.numel())
    copies = max(2, math.ceil(3 * MALL_BYTES / nbytes))
    caches = [(kc, ks, vc, vs)] + [tuple(t.clone() for t in (kc, ks, vc, vs))
                                   for _ in range(copies - 1)]
    ws = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D, splits)
    out = torch.empty_like(qd)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def call(i):
        c = caches[i % copies]
        st = lib.kvq_attend(P(qd), P(c[0]), P(c[1]), P(c[2]), P(c[3]), w.B, w.Hq, w.Hkv, w.R, w.N,
                            w.D, bits, group, 0.0, splits, P(ws), ws.numel(), P(out), stream)
        if st != 0:
            raise RuntimeError(f"kvq_attend: status {st}")

    heads = w.B * w.Hkv
    grid = (splits or lib_auto_splits(w)) * heads  # an upper bound: rows a launch wrote are kept
    waves_per_wg = 8 if kernel in (0, 2) else 4
    nw = min(PHASE_WAVES, grid * waves_per_wg)
    buf = np.zeros(PHASE_WAVES * PHASE_MARKS, np.uint64)
    for i in range(2 * copies):
        call(i)
    torch.cuda.synchronize()
    rec, spans, recorded = [], [], 0
    for b in range(batches):
        for i in range(per_batch):
            call(b * per_batch + i)
        torch.cuda.synchronize()
        st = lib.kvq_phase_trace_fetch(kernel, buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes)
        if st != 0:
            raise RuntimeError(f"kvq_phase_trace_fetch: status {st}")
        t = buf[:nw * PHASE_MARKS].reshape(nw, PHASE_MARKS).astype(np.int64)
        t = t[(t[:, 0] != 0) & (t[:, 7] != 0)]  # rows a launch wrote (the array starts zeroed)
        recorded = t.shape[0]
        t0 = t[:, 0].min()
        x = (t - t0) * 0.01  # us since the launch's first wave started
        # a mark outside its wave's [start, end] was not reached in this launch
        bad = (x < x[:, :1]) | (x > x[:, 7:8])
        x = np.where(bad, np.nan, x)
        rec.append(x)
        spans.append(np.nanmax(x[:, 7]))
    x = np.concatenate(rec)
    print(f"# {workload} {bits}-bit g{group}: kernel {KERNELS[kernel]}, "
          f"{splits if splits else 'automatic'} splits, {recorded // waves_per_wg} workgroups x "
          f"{waves_per_wg} waves recorded; {batches} batches of {per_batch} back-to-back launches "
          f"over {copies} cache copies, the last launch of each batch recorded")
    print()
    print("| mark | p10 (us) | p50 (us) | p90 (us) | max (us) |")
    print("|---|---|---|---|---|")
    for j, name in enumerate(MARKS):
        c = x[:, j][~np.isnan(x[:, j])]
        if c.size:
            print(f"| {name} | {np.percentile(c, 10):.2f} | {np.percentile(c, 50):.2f} | "
                  f"{np.percentile(c, 90):.2f} | {c.max():.2f} |")
    print()
    print("| step (per wave) | p10 (us) | p50 (us) | p90 (us) |")
    print("|---|---|---|---|")
    prev = 0
    for j in range(1, PHASE_MARKS):
        if np.all(np.isnan(x[:, j])):
            continue
        d = x[:, j] - x[:, prev]
        d = d[~np.isnan(d)]
        print(f"| {MARKS[prev]} -> {MARKS[j]} | {np.percentile(d, 10):.2f} | "
              f"{np.percentile(d, 50):.2f} | {np.percentile(d, 90):.2f} |")
        prev = j
    print()
    print(f"launch span (first wave start -> last wave end): median {np.median(spans):.2f} us, "
          f"min {np.min(spans):.2f}, max {np.max(spans):.2f}")


def lib_auto_splits(w) -> int:
    return kvq.auto_splits(w.B, w.Hkv, w.N)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="gqa_n4096", choices=["gqa_n4096", "gqa_n32768"])
    ap.add_argument("--splits", type=int, default=-1, help="-1: the workload's default, 0: auto")
    ap.add_argument("--batches", type=int, default=12)
    ap.add_argument("--per-batch", type=int, default=20)
    ap.add_argument("--format", default="", help="bits,group (default: the workload's own)")
    args = ap.parse_args()
    fmt = tuple(int(x) for x in args.format.split(",")) if args.format else None
    run(args.workload, args.splits, args.batches, args.per_batch, fmt)


if __name__ == "__main__":
    main()
