"""Pins of the oracle's mixed cache (``attend_window``): the oldest N - W
tokens packed, the most recent W in float32.

Pinned by its two ends and by its decoded cache, none of which re-states its
steps: W = 0 is the packed path (``attend_packed`` over all N), W = N the
float32 path (``attend_dense`` on the raw K/V); for 0 < W < N the result is
attention over [decoded packed prefix ; raw window], where the prefix is
decoded from a cache grown to N - W tokens (``cache_after`` read back with
the layout formula of the growing-cache pins), and the window must help on
inputs whose attention leans on the recent tokens."""
import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import Workload, make_qkv

from test_oracle_cache import readback


def _qkv(n, d, seed, dist="clean"):
    w = Workload("win", 1, 2, 1, 4, n, d, ((4, 8),))
    return make_qkv(w, seed, dist)


@pytest.mark.parametrize("bits,group", [(4, 8), (8, 32)])
def test_window_ends(bits, group):
    q, k, v = _qkv(70, 16, 0)
    kc, ks = O.pack_k(k, bits, group)
    vc, vs = O.pack_v(v, bits, group)
    assert np.array_equal(O.attend_window(q, k, v, 0, bits, group),
                          O.attend_packed(q, kc, ks, vc, vs, 70, bits, group))
    assert np.array_equal(O.attend_window(q, k, v, 70, bits, group), O.attend_dense(q, k, v))


@pytest.mark.parametrize("w", [1, 7, 33])
def test_window_is_grown_cache_plus_raw_tail(w):
    n, d, bits, group = 70, 16, 4, 8
    q, k, v = _qkv(n, d, 1)
    npk = n - w
    kc, ks, vc, vs = O.cache_after(k, v, npk, npk, bits, group)
    k_codes, k_sc, v_codes, v_sc = readback(kc, ks, vc, vs, npk, d, bits, group)
    qmax = 7
    k_hat = np.concatenate([((k_codes - qmax) * k_sc).astype(np.float32), k[..., npk:, :]], -2)
    v_hat = np.concatenate([((v_codes - qmax) * v_sc).astype(np.float32), v[..., npk:, :]], -2)
    want = O.attend_dense(q, k_hat, v_hat)
    assert np.max(np.abs(O.attend_window(q, k, v, w, bits, group) - want)) <= 1e-12


def test_recent_window_helps_late_biased_attention():
    """Keys biased toward the last 16 tokens: keeping those in float32
    removes most of their quantization error; for the early bias it need
    not (the study's question on the page)."""
    errs = {}
    for dist in ("late", "early"):
        e0 = e16 = 0.0
        for seed in (0, 1, 2):
            q, k, v = _qkv(512, 32, seed, dist)
            ref = O.attend_dense(q, k, v)
            e0 += O.rel_l2(O.attend_window(q, k, v, 0, 4, 32), ref)
            e16 += O.rel_l2(O.attend_window(q, k, v, 16, 4, 32), ref)
        errs[dist] = (e0, e16)
    assert errs["late"][1] < 0.5 * errs["late"][0]
    assert errs["early"][1] > 0.8 * errs["early"][0]


def test_causal_window():
    q, k, v = _qkv(40, 16, 2)
    out = O.attend_window(q, k, v, 10, 4, 8, causal=True)
    assert np.isfinite(out).all()
    assert np.array_equal(O.attend_window(q, k, v, 40, 4, 8, causal=True),
                          O.attend_dense(q, k, v, causal=True))
