"""Helpers shared by the GPU tests: device transfer and oracle-side packing
of the same seeded inputs the GPU sees."""
import sys

import numpy as np

from oracle import kvq_oracle as O


def announce(msg: str) -> None:
    """Name the GPU case on stdout before it runs (survives a lost box)."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def oracle_pack(k, v, bits, group):
    kc, ks = O.pack_k(k, bits, group)
    vc, vs = O.pack_v(v, bits, group)
    return kc, ks, vc, vs


def oracle_store(k, v, bits, group):
    """The oracle's packing of k, v in the library's block byte order."""
    n, d = k.shape[-2], k.shape[-1]
    kc, ks, vc, vs = oracle_pack(k, v, bits, group)
    return O.store_k(kc, ks, n, d, bits, group) + O.store_v(vc, vs, n, d, bits, group)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
