"""Pins of the oracle's growing cache (``cache_after``): the packed cache
after n appended tokens, laid out for a larger capacity.

Reading ([RL] "prefill and decode"; [KPG] "why grouping needs both direction
and length"): the cache of n tokens is the packed tensor of those n tokens,
short groups zero-padded.  Pinned three ways, none of which re-calls
``cache_after``'s own steps:
  * at n = capacity it is plain packing of the whole input;
  * its bytes, read back with the byte formula the C header states (written
    out here index by index), give the prefix's codes and scales, and the
    zero code / scale 1 everywhere past n;
  * a token-by-token append (a new token's V row quantized alone, the open K
    group requantized from its raw values) agrees with it at every n.
"""
import numpy as np
import pytest

from oracle import kvq_oracle as O

QMAX = {4: 7, 8: 127}


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def readback(kc, ks, vc, vs, cap, d, bits, group):
    """Stored codes [..., cap, D] and per-element scales of K and V, read
    from the block layout with the header's byte formula."""
    lead = kc.shape[:-2]
    kcols = 32 * bits // 8
    d8 = -(-d // 8)
    dpad = -(-d // group) * group
    vcols = dpad * bits // 8
    k_codes = np.zeros(lead + (cap, d), np.int64)
    v_codes = np.zeros(lead + (cap, d), np.int64)
    k_sc = np.zeros(lead + (cap, d), np.float32)
    v_sc = np.zeros(lead + (cap, d), np.float32)
    kflat = kc.reshape(lead + (-1,))
    vflat = vc.reshape(lead + (-1,))
    vsc = vs.reshape(lead + (-1, dpad // group, 32))
    for t in range(cap):
        blk, tl = divmod(t, 32)
        for c in range(d):
            j = tl // 2 if bits == 4 else tl
            kb = kflat[..., blk * d8 * kcols * 8 + ((c // 8) * kcols + j) * 8 + c % 8]
            vcol = c // 2 if bits == 4 else c
            vb = vflat[..., blk * 4 * vcols * 8 + ((tl // 8) * vcols + vcol) * 8 + tl % 8]
            if bits == 4:
                kb = (kb >> 4) if t % 2 else (kb & 15)
                vb = (vb >> 4) if c % 2 else (vb & 15)
            k_codes[..., t, c] = kb
            v_codes[..., t, c] = vb
            k_sc[..., t, c] = ks[..., t // group, c]
            v_sc[..., t, c] = vsc[..., blk, c // group, tl]
    return k_codes, k_sc, v_codes, v_sc


@pytest.mark.parametrize("bits,group", [(4, 8), (4, 32), (8, 6)])
def test_full_capacity_is_plain_packing(bits, group):
    k, v = _rand((2, 3, 45, 12), 0), _rand((2, 3, 45, 12), 1)
    got = O.cache_after(k, v, 45, 45, bits, group)
    want = (*O.store_k(*O.pack_k(k, bits, group), 45, 12, bits, group),
            *O.store_v(*O.pack_v(v, bits, group), 45, 12, bits, group))
    for a, b in zip(got, want):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("n", [0, 1, 7, 8, 31, 32, 33])
@pytest.mark.parametrize("bits,group", [(4, 8), (4, 32), (8, 6)])
def test_prefix_codes_and_empty_positions(n, bits, group):
    cap, d = 40, 10
    k, v = _rand((1, 2, cap, d), 2), _rand((1, 2, cap, d), 3)
    kc, ks, vc, vs = O.cache_after(k, v, n, cap, bits, group)
    assert kc.shape[-2] == -(-cap // 32) and ks.shape[-2] == -(-cap // group)
    k_codes, k_sc, v_codes, v_sc = readback(kc, ks, vc, vs, cap, d, bits, group)
    qmax = QMAX[bits]
    # past n: the zero code everywhere, scale 1 for V and for K groups holding no token < n
    assert (k_codes[..., n:, :] == qmax).all() and (v_codes[..., n:, :] == qmax).all()
    assert (v_sc[..., n:, :] == 1.0).all()
    first_empty = -(-n // group) * group
    assert (k_sc[..., first_empty:, :] == 1.0).all()
    if n:
        # the prefix: same codes and scales as packing the n tokens alone
        pk, pks, pv, pvs = (*O.store_k(*O.pack_k(k[..., :n, :], bits, group), n, d, bits, group),
                            *O.store_v(*O.pack_v(v[..., :n, :], bits, group), n, d, bits, group))
        want = readback(pk, pks, pv, pvs, n, d, bits, group)
        for got, w in zip((k_codes, k_sc, v_codes, v_sc), want):
            assert np.array_equal(got[..., :n, :], w)
        # the open K group's scale is max |x| / qmax over its tokens below n
        g0 = (n - 1) // group * group
        amax = np.abs(k[..., g0:n, :]).max(axis=-2)
        want_s = np.where(amax == 0, np.float32(1), amax / np.float32(qmax)).astype(np.float32)
        assert np.array_equal(k_sc[..., g0, :], want_s)


def _quant(x, bits):
    """Scale and stored codes of one group (last axis), in float32."""
    qmax = np.float32(QMAX[bits])
    s = (np.abs(x).max(axis=-1, keepdims=True) / qmax).astype(np.float32)
    s = np.where(s == 0, np.float32(1), s)
    c = np.clip(np.rint(x / s), -qmax, qmax).astype(np.int64) + QMAX[bits]
    return s, c


@pytest.mark.parametrize("bits,group", [(4, 8), (4, 4), (8, 6)])
def test_token_by_token_append(bits, group):
    cap, d = 21, 6
    k, v = _rand((1, 2, cap, d), 4), _rand((1, 2, cap, d), 5)
    qmax = QMAX[bits]
    dpad = -(-d // group) * group
    kcode = np.full((1, 2, cap, d), qmax, np.int64)
    vcode = np.full((1, 2, cap, d), qmax, np.int64)
    ksc = np.ones((1, 2, cap, d), np.float32)
    vsc = np.ones((1, 2, cap, d), np.float32)
    for n in range(1, cap + 1):
        t = n - 1
        # V: the new token's row, feature groups zero-padded to dpad
        row = np.zeros((1, 2, dpad), np.float32)
        row[..., :d] = v[..., t, :]
        s, c = _quant(row.reshape(1, 2, dpad // group, group), bits)
        vcode[..., t, :] = c.reshape(1, 2, dpad)[..., :d]
        vsc[..., t, :] = np.repeat(s[..., 0], group, axis=-1)[..., :d]
        # K: requantize the open group (tokens g0 .. t of each channel)
        g0 = t // group * group
        grp = np.zeros((1, 2, d, group), np.float32)
        grp[..., : t - g0 + 1] = np.swapaxes(k[..., g0:t + 1, :], -1, -2)
        s, c = _quant(grp, bits)
        span = min(group, cap - g0)
        kcode[..., g0:g0 + span, :] = np.swapaxes(c, -1, -2)[..., :span, :]
        ksc[..., g0:g0 + span, :] = np.swapaxes(np.broadcast_to(s, grp.shape), -1, -2)[..., :span, :]
        got = readback(*O.cache_after(k, v, n, cap, bits, group), cap, d, bits, group)
        for a, b in zip(got, (kcode, ksc, vcode, vsc)):
            assert np.array_equal(a, b), n


def test_attention_over_the_prefix_ignores_the_rest():
    """Attending the first n tokens of a capacity cache equals attending a
    cache packed from those n tokens (the positions past n never count)."""
    k, v = _rand((1, 2, 50, 16), 6), _rand((1, 2, 50, 16), 7)
    q = _rand((1, 4, 2, 16), 8)
    n = 37
    kc, ks = O.pack_k(k[..., :n, :], 4, 8)
    vc, vs = O.pack_v(v[..., :n, :], 4, 8)
    want = O.attend_packed(q, kc, ks, vc, vs, n, 4, 8)
    # the padded cache's first n decoded tokens are the same
    kp = np.zeros_like(k)
    kp[..., :n, :] = k[..., :n, :]
    k_hat = O.dequant_k(*O.pack_k(kp, 4, 8), k.shape, 4, 8)[..., :n, :]
    k_ref = O.dequant_k(kc, ks, (1, 2, n, 16), 4, 8)
    assert np.array_equal(k_hat, k_ref)
    assert np.isfinite(want).all()
