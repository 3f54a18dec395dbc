"""Pins of the oracle's causal chunk: R queries that are the sequence's last
R positions, query i reading tokens j <= n - R + i ([RL] "prefill and
decode"; masked positions and rows with no legal key per [RL] "why
FlashAttention need not keep the whole heat map").

Pinned without re-stating the mask: a per-query brute force over the
visible prefix with scalar math.exp, the R = 1 reduction to the unmasked
path, zeros for rows with no legal key, and the blocked recurrence (blocks
of 7, some wholly masked for some rows) equal to the dense result."""
import math

import numpy as np
import pytest

from oracle import kvq_oracle as O


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def brute_row(qv, keys, vals, scale):
    """softmax(q.k * scale) v over the given keys, scalar loops in float64."""
    s = [scale * sum(float(a) * float(b) for a, b in zip(qv, k)) for k in keys]
    if not s:
        return [0.0] * len(qv)
    mx = max(s)
    w = [math.exp(x - mx) for x in s]
    tot = sum(w)
    return [sum(wi * float(v[f]) for wi, v in zip(w, vals)) / tot for f in range(len(vals[0]))]


@pytest.mark.parametrize("n,r,hq,hkv", [(9, 3, 2, 1), (5, 4, 4, 2), (2, 4, 1, 1), (1, 1, 1, 1)])
def test_causal_matches_per_query_brute_force(n, r, hq, hkv):
    d = 5
    q = _rand((1, hq, r, d), 0)
    k = _rand((1, hkv, n, d), 1)
    v = _rand((1, hkv, n, d), 2)
    scale = 1.0 / math.sqrt(d)
    got = O.attend_dense(q, k, v, causal=True)
    for h in range(hq):
        kv = h // (hq // hkv)
        for i in range(r):
            last = n - r + i                      # position of query i
            keys = [k[0, kv, j] for j in range(n) if j <= last]
            vals = [v[0, kv, j] for j in range(n) if j <= last]
            want = brute_row(q[0, h, i], keys, vals, scale)
            assert np.allclose(got[0, h, i], want, rtol=0, atol=1e-12), (h, i)


def test_single_query_is_unmasked():
    q, k, v = _rand((2, 4, 1, 16), 3), _rand((2, 2, 37, 16), 4), _rand((2, 2, 37, 16), 5)
    assert np.array_equal(O.attend_dense(q, k, v, causal=True), O.attend_dense(q, k, v))


def test_rows_with_no_key_are_zero():
    q, k, v = _rand((1, 2, 6, 8), 6), _rand((1, 1, 2, 8), 7), _rand((1, 1, 2, 8), 8)
    out = O.attend_dense(q, k, v, causal=True)
    assert np.isfinite(out).all()
    assert (out[:, :, :4] == 0).all()             # queries 0..3 sit before token 0
    assert (np.abs(out[:, :, 4:]) > 0).any()
    assert O.causal_mask(2, 6).sum(axis=1).tolist() == [0, 0, 0, 0, 1, 2]


@pytest.mark.parametrize("n,r", [(30, 8), (6, 8), (64, 4)])
def test_blocked_recurrence_equals_dense_under_the_mask(n, r):
    q, k, v = _rand((1, 4, r, 16), 9), _rand((1, 2, n, 16), 10), _rand((1, 2, n, 16), 11)
    dense = O.attend_dense(q, k, v, causal=True)
    blocked = O.attend_blocked(q, k, v, 7, causal=True)
    assert np.isfinite(blocked).all()
    assert np.max(np.abs(dense - blocked)) <= 1e-10


def test_split_merge_under_the_mask():
    """Splits composed with the same rescale ([RL] "two stops of the online
    accumulation"), where whole splits see no legal key for some rows."""
    n, r = 40, 8
    q, k, v = _rand((1, 2, r, 8), 12), _rand((1, 1, n, 8), 13), _rand((1, 1, n, 8), 14)
    dense = O.attend_dense(q, k, v, causal=True)
    rows = q.reshape(1, 1, 2 * r, 8).astype(np.float64)
    vis = np.tile(O.causal_mask(n, r), (2, 1))
    s = np.where(vis, (rows @ np.swapaxes(k.astype(np.float64), -1, -2)) / math.sqrt(8), -np.inf)
    # two blocks: tokens 0..34 and 35..39 (the second is empty for rows 0..2)
    out, _ = O.merge_blocks([s[..., :35], s[..., 35:]],
                            [v[..., None, :35, :], v[..., None, 35:, :]])
    assert np.max(np.abs(out.reshape(dense.shape) - dense)) <= 1e-12
