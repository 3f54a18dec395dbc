"""Accuracy of the packed formats, measured on the GPU.

"KV分组打包：4-bit到底省了多少？" (huhohoo.com/docs/llm/kv-packed-groups),
"accuracy and space on the same input": for each input, the relative L2
error of the attention output over the quantized cache against the output
over the float32 cache, ||O_q - O_f32||_F / ||O_f32||_F over the input's
whole output, then the mean over inputs; set against the packed bytes per
KV head.  The page runs it on small NumPy inputs (N = 128 / 512, D = 32,
four queries, clean and +4 sigma biased keys, three seeds); this runs the
same recipe through the library's kernels (pack, fused attend, and the
float32-cache attend as the reference) at any size.

    python -m quantized_kv_cache_attend_amd.accuracy [--n 128 512 4096] [--d 32 128]
        [--window 0 16 64]

prints one markdown table (mean relative L2 per format, length, head dim and
distribution) and, with --json, the per-input values.  --window adds the
mixed cache the same page announces as its next study ("exercises and
common mistakes": high precision kept for the most recent tokens): the last
W tokens in float32 (kvq_attend_window), the rest packed.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

FORMATS = ((4, 8), (4, 32), (8, 8), (8, 32))
DISTS = ("clean", "early", "late")


def rel_l2(approx: np.ndarray, ref: np.ndarray) -> float:
    """||approx - ref||_F / ||ref||_F in float64 over one input's output."""
    a = np.asarray(approx, np.float64)
    r = np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - r) / np.linalg.norm(r))


def packed_bytes_per_head(n: int, d: int, bits: int, group: int) -> int:
    """Code bytes + float32 scales of one KV head's packed K and V (the
    page's payload without the two shape records)."""
    npad = -(-n // group) * group
    dpad = -(-d // group) * group
    return (d * npad + n * dpad) * bits // 8 + 4 * (d * npad // group + n * dpad // group)


def study(lengths, dims, seeds=(0, 1, 2), dists=DISTS, formats=FORMATS, queries=4,
          device="cuda", windows=(0,)):
    """Per-input relative L2 errors on the GPU.  Returns a list of dicts
    (n, d, dist, seed, bits, group, window, rel_l2, packed_bytes); window W > 0:
    the last W tokens stay float32 (packed_bytes then counts them at 4 bytes
    per element)."""
    import torch

    import quantized_kv_cache_attend_amd as kvq
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import Workload, make_qkv

    rows = []
    for n in lengths:
        for d in dims:
            for dist in dists:
                for seed in seeds:
                    w = Workload("acc", 1, 1, 1, queries, n, d, formats)
                    q, k, v = make_qkv(w, seed, dist)
                    qd, kd, vd = (torch.from_numpy(a).to(device) for a in (q, k, v))
                    ref = kvq.attend_f32(qd, kd, vd).cpu().numpy()
                    for bits, group in formats:
                        for win in windows:
                            if win >= n:
                                continue
                            npk = n - win
                            kc, ks = kvq.pack_k(kd[:, :, :npk].contiguous(), bits, group)
                            vc, vs = kvq.pack_v(vd[:, :, :npk].contiguous(), bits, group)
                            if win:
                                out = kvq.attend_window(qd, kc, ks, vc, vs,
                                                        kd[:, :, npk:].contiguous(),
                                                        vd[:, :, npk:].contiguous(), npk, bits,
                                                        group)
                            else:
                                out = kvq.attend(qd, kc, ks, vc, vs, n, bits, group)
                            nbytes = packed_bytes_per_head(npk, d, bits, group) + 8 * win * d
                            rows.append({"n": n, "d": d, "dist": dist, "seed": seed,
                                         "bits": bits, "group": group, "window": win,
                                         "rel_l2": rel_l2(out.cpu().numpy(), ref),
                                         "packed_bytes": nbytes})
    return rows


def table(rows) -> str:
    """Mean over seeds, one line per (n, d, dist, window), one column per format."""
    fmts = sorted({(r["bits"], r["group"]) for r in rows}, key=lambda f: (f[0], f[1]))
    keys = sorted({(r["n"], r["d"], r["dist"], r["window"]) for r in rows},
                  key=lambda k: (k[0], k[1], DISTS.index(k[2]) if k[2] in DISTS else 9, k[3]))
    head = "| N | D | keys | float32 window | " + " | ".join(f"{b}-bit g{g}" for b, g in fmts) + " |"
    lines = [head, "|" + "---|" * (4 + len(fmts))]
    for n, d, dist, win in keys:
        cells = []
        for b, g in fmts:
            vals = [r["rel_l2"] for r in rows
                    if (r["n"], r["d"], r["dist"], r["window"], r["bits"], r["group"]) ==
                    (n, d, dist, win, b, g)]
            cells.append(f"{100 * np.mean(vals):.3f} %" if vals else "-")
        lines.append(f"| {n} | {d} | {dist} | {win} | " + " | ".join(cells) + " |")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--n", type=int, nargs="+", default=[128, 512, 4096, 32768])
    ap.add_argument("--d", type=int, nargs="+", default=[32, 128])
    ap.add_argument("--seeds", type=int, nargs="+", default=[0, 1, 2])
    ap.add_argument("--window", type=int, nargs="+", default=[0],
                    help="float32 windows of the most recent tokens (0: fully packed)")
    ap.add_argument("--json", help="write the per-input values here")
    args = ap.parse_args(argv)
    rows = study(args.n, args.d, tuple(args.seeds), windows=tuple(args.window))
    print(table(rows))
    if args.json:
        with open(args.json, "w", encoding="utf-8") as f:
            json.dump(rows, f, indent=1)


if __name__ == "__main__":
    main()
