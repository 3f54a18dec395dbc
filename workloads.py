"""Seeded synthetic inputs for the packed-KV attention workloads.

This module only draws random numbers and shapes them; it contains none of
the method's arithmetic (no quantization, packing or attention).  Both the
oracle-side tests and the GPU-side tests and benchmark take their inputs from
here, so the two sides see identical float32 Q, K and V.

Workloads (the pages measure fixed synthetic arrays, never a dataset):

  single_n128   1 head, N=128,  D=32, 4 queries, 4-bit group 32, block 32
  single_n512   1 head, N=512,  D=32, 4 queries, four formats (g8/g32 x 4/8-bit)
                plus the float32-cache path, block 32
  single_n1024  1 head, N=1024, D=32, 8 queries, 4-bit group 8, block 7,
                three score distributions (clean, early-biased, late-biased)
  gqa_n4096     batch 8, n=4096, Hq=32 / Hkv=8, d=128, 1 query per head,
                4-bit group 32 (one layer)
  gqa_n32768    batch 16, n=32768, Hq=64 / Hkv=8, d=128, 4 queries per head,
                4-bit group 32, K channels scaled log-uniformly over [0.1, 10],
                16 KV splits

Recipe: ``numpy.random.default_rng(seed)`` (PCG64), draws in the order Q, K,
V (then the per-channel K magnitudes), each ``standard_normal`` in float32.
Seeds 0, 1, 2.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

SEEDS = (0, 1, 2)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    R: int
    N: int
    D: int
    formats: tuple          # ((bits, group), ...)
    block: int = 32         # block length of the oracle's blocked path
    dists: tuple = ("clean",)
    k_channel_scale: bool = False
    num_splits: int = 0     # 0 = let the library choose

    @property
    def rows_per_kv_head(self) -> int:
        return (self.Hq // self.Hkv) * self.R


WORKLOADS = {
    w.name: w
    for w in (
        Workload("single_n128", 1, 1, 1, 4, 128, 32, ((4, 32),)),
        Workload("single_n512", 1, 1, 1, 4, 512, 32, ((4, 8), (4, 32), (8, 8), (8, 32))),
        Workload("single_n1024", 1, 1, 1, 8, 1024, 32, ((4, 8),), block=7,
                 dists=("clean", "early", "late")),
        Workload("gqa_n4096", 8, 32, 8, 1, 4096, 128, ((4, 32),)),
        Workload("gqa_n32768", 16, 64, 8, 4, 32768, 128, ((4, 32),),
                 k_channel_scale=True, num_splits=16),
    )
}

# Tokens whose keys get the +4 sigma bias in the early / late distributions.
BIAS_TOKENS = 16
BIAS_SIGMAS = 4.0


def make_qkv(w: Workload, seed: int, dist: str = "clean", n: int | None = None):
    """Return float32 ``q [B,Hq,R,D]``, ``k [B,Hkv,N,D]``, ``v [B,Hkv,N,D]``.

    ``n`` overrides the token count (for reduced-size test cases of the same
    recipe).

    ``dist``:
      * ``clean``: i.i.d. N(0, 1).
      * ``early`` / ``late``: the keys of the first / last 16 tokens are moved
        along the mean query direction qbar so that the mean score of those
        tokens over the queries rises by 4 standard deviations of the clean
        scores: k_j += alpha * qbar with alpha = 4 * sigma_s * sqrt(D) / |qbar|^2,
        sigma_s the std of the clean scores q.k/sqrt(D).
    With ``k_channel_scale`` every channel d of KV head h is multiplied by
    sigma[h, d] = 10**U(-1, 1) (log-uniform on [0.1, 10], shared over the
    batch).
    """
    n = w.N if n is None else int(n)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((w.B, w.Hq, w.R, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, n, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, n, w.D), dtype=np.float32)
    if w.k_channel_scale:
        sigma = (10.0 ** rng.uniform(-1.0, 1.0, size=(w.Hkv, w.D))).astype(np.float32)
        k *= sigma[None, :, None, :]
    if dist != "clean":
        if dist not in ("early", "late"):
            raise ValueError(f"unknown distribution {dist!r}")
        rep = w.Hq // w.Hkv
        for b in range(w.B):
            for h in range(w.Hkv):
                qs = q[b, h * rep:(h + 1) * rep].reshape(-1, w.D).astype(np.float64)
                kk = k[b, h].astype(np.float64)
                sigma_s = float(np.std(qs @ kk.T / math.sqrt(w.D)))
                qbar = qs.mean(axis=0)
                alpha = BIAS_SIGMAS * sigma_s * math.sqrt(w.D) / float(qbar @ qbar)
                idx = slice(0, BIAS_TOKENS) if dist == "early" else slice(n - BIAS_TOKENS, n)
                k[b, h, idx] = (kk[idx] + alpha * qbar).astype(np.float32)
    return q, k, v


def make_crafted(kind: str, seed: int = 0):
    """Small crafted float32 arrays for edge cases of the quantizer.

    ``ragged``  35 x 13 Gaussian matrix (not divisible by 8 or 32).
    ``zeros``   an all-zero 64 x 32 matrix.
    ``ties``    a 2 x 32 matrix whose groups hold exact .5 quotients.
    ``tiny``    a 4 x 32 matrix of subnormal-sized values.
    """
    rng = np.random.default_rng(seed)
    if kind == "ragged":
        return rng.standard_normal((35, 13), dtype=np.float32)
    if kind == "zeros":
        return np.zeros((64, 32), dtype=np.float32)
    if kind == "ties":
        row = np.array([7, 0.5, 1.5, 2.5, -2.5, 3.5, -3.5, 4.5, -4.5, 5.5, -5.5, 6.5, -6.5,
                        -0.5, -1.5, 0, 1, 2, 3, 4, 5, 6, -1, -2, -3, -4, -5, -6, -7, 0.25,
                        -0.75, 1.25], dtype=np.float32)
        return np.stack([row, -row])
    if kind == "tiny":
        x = rng.standard_normal((4, 32), dtype=np.float32) * np.float32(1e-39)
        # a row of at most 3 smallest subnormals: max|x|/7 underflows to zero
        x[1] = rng.integers(-3, 4, size=32).astype(np.float32) * np.float32(2.0 ** -149)
        x[1, 0] = np.float32(3 * 2.0 ** -149)
        return x.astype(np.float32)
    raise ValueError(kind)
