"""GPU parity of the matrix-core kernels on 8-bit codes (group 32, D = 128):
one code byte per element, offset 127, the same block algebra as 4-bit.
Against the float64 oracle (<= 1e-4) on ragged token counts, 1..32 query
rows per KV head (both kernels, one and two row tiles), concentrated
softmaxes, large K scales, the causal chunk, a cache laid out for a larger
capacity, the fused recent-token window and the 8 x 4096-token cache shape;
and against the general kernel on the same problems (<= 2e-5)."""
import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import WORKLOADS, Workload, make_qkv

from gpu_helpers import announce, dev, host, max_abs, oracle_pack

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")

TOL = 1e-4
SPLIT_TOL = 2e-5
BITS, GROUP = 8, 32


def _cache(k, v):
    gkc, gks = kvq.pack_k(dev(k), BITS, GROUP)
    gvc, gvs = kvq.pack_v(dev(v), BITS, GROUP)
    return gkc, gks, gvc, gvs


def _oracle(q, k, v, causal=False):
    kc, ks, vc, vs = oracle_pack(k, v, BITS, GROUP)
    return O.attend_packed(q, kc, ks, vc, vs, k.shape[2], BITS, GROUP, causal=causal)


# (Hq, Hkv, R): rows per KV head 4 (4-row kernel), 1, 5 and 16 (32-row kernel,
# one tile), 18 and 32 (two tiles).
SHAPES = [(8, 2, 1), (1, 1, 1), (5, 1, 1), (16, 2, 2), (6, 1, 3), (8, 1, 4)]


@pytest.mark.parametrize("hq,hkv,r", SHAPES)
@pytest.mark.parametrize("n", [1, 35, 1021, 4097])
def test_mfma8_ragged_and_gqa_shapes(hq, hkv, r, n):
    w = Workload("mfma8", 2, hq, hkv, r, n, 128, ((BITS, GROUP),))
    q, k, v = make_qkv(w, 21)
    announce(f"mfma 8-bit hq={hq} hkv={hkv} r={r} n={n}")
    want = _oracle(q, k, v)
    cache = _cache(k, v)
    qd = dev(q)
    general = host(kvq.attend(qd, *cache, n, BITS, GROUP, num_splits=3, variant="valu"))
    for splits in (1, 3, 0, 64):
        got = host(kvq.attend(qd, *cache, n, BITS, GROUP, num_splits=splits, variant="mfma"))
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))
        assert max_abs(got, general) <= SPLIT_TOL, (splits, max_abs(got, general))


@pytest.mark.parametrize("hq,hkv,r", [(16, 4, 1), (16, 2, 4)])
@pytest.mark.parametrize("dist,scale_k", [("clean", False), ("clean", True), ("early", True),
                                          ("late", True)])
def test_mfma8_peaky_and_channel_scaled(hq, hkv, r, dist, scale_k):
    """Keys biased +4 sigma on 16 tokens and log-uniform K channel
    magnitudes concentrate the softmax."""
    w = Workload("peaky8", 2, hq, hkv, r, 4096, 128, ((BITS, GROUP),), k_channel_scale=scale_k)
    q, k, v = make_qkv(w, 22, dist)
    announce(f"mfma 8-bit peaky hq={hq} hkv={hkv} r={r} dist={dist} scale_k={scale_k}")
    want = _oracle(q, k, v)
    cache = _cache(k, v)
    for splits in (1, 0):
        got = host(kvq.attend(dev(q), *cache, w.N, BITS, GROUP, num_splits=splits,
                              variant="mfma"))
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


@pytest.mark.parametrize("hq,r", [(4, 1), (16, 2)])
def test_mfma8_large_k_scales(hq, r):
    """K scales (max |k| / 127) of about 90, past the bound at which a block's
    scales are first divided by a power of two, and one group of small
    scales among them."""
    w = Workload("bigk8", 1, hq, 1, r, 1000, 128, ((BITS, GROUP),))
    q, k, v = make_qkv(w, 23)
    k = (k * np.float32(3000.0)).astype(np.float32)
    k[0, 0, 500:532] *= np.float32(0.001)
    announce(f"mfma 8-bit large K scales hq={hq} r={r}")
    # A temperature that keeps the scores near the size the other tests see
    # (float32 scores of magnitude ~3e4 carry ~1e-3 rounding on any kernel).
    want = O.attend_packed(q, *oracle_pack(k, v, BITS, GROUP), w.N, BITS, GROUP, sm_scale=1e-3)
    cache = _cache(k, v)
    for splits in (1, 0):
        got = host(kvq.attend(dev(q), *cache, w.N, BITS, GROUP, num_splits=splits,
                              variant="mfma", sm_scale=1e-3))
        assert np.isfinite(got).all()
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


@pytest.mark.parametrize("B,hq,hkv,r,n", [
    (2, 8, 8, 2, 4097),     # 2 rows: 4-row kernel
    (1, 2, 2, 4, 3),        # 4-row kernel, N < R: rows without a key
    (2, 8, 2, 4, 100),      # 16 rows: one tile
    (2, 4, 1, 8, 70),       # 32 rows, the mask spans two blocks
])
def test_mfma8_causal(B, hq, hkv, r, n):
    w = Workload("causal8", B, hq, hkv, r, n, 128, ((BITS, GROUP),))
    q, k, v = make_qkv(w, 24)
    announce(f"mfma 8-bit causal B={B} hq={hq} hkv={hkv} R={r} N={n}")
    want = _oracle(q, k, v, causal=True)
    cache = _cache(k, v)
    empty = O.causal_mask(n, r).sum(axis=1) == 0
    for splits in (1, 3, 0, 64):
        got = host(kvq.attend(dev(q), *cache, n, BITS, GROUP, num_splits=splits, variant="mfma",
                              causal=True))
        assert np.isfinite(got).all(), splits
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))
        assert (got[:, :, empty] == 0).all()


@pytest.mark.parametrize("hq,hkv,r", [(8, 2, 1), (16, 2, 2)])
def test_mfma8_cache_prefix(hq, hkv, r):
    """A cache laid out for 1100 tokens and grown by appends: attending its
    first n tokens equals attending a cache packed from those n alone, bit
    for bit, and the oracle within 1e-4."""
    import torch
    cap, D = 1100, 128
    w = Workload("cache8", 2, hq, hkv, r, cap, D, ((BITS, GROUP),))
    q, k, v = make_qkv(w, 25)
    announce(f"mfma 8-bit cache prefix rows={hq // hkv * r}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    cache = kvq.new_cache(2, hkv, cap, D, BITS, GROUP)
    n = 0
    for t in (1, 30, 2, 500, 488, 1):
        kvq.append(kd[:, :, n:n + t].contiguous(), vd[:, :, n:n + t].contiguous(), n, cache, cap,
                   BITS, GROUP)
        n += t
        got = kvq.attend(qd, *cache[:4], n, BITS, GROUP, variant="mfma", capacity=cap)
        fk, fks = kvq.pack_k(kd[:, :, :n].contiguous(), BITS, GROUP)
        fv, fvs = kvq.pack_v(vd[:, :, :n].contiguous(), BITS, GROUP)
        fresh = kvq.attend(qd, fk, fks, fv, fvs, n, BITS, GROUP, variant="mfma")
        torch.cuda.synchronize()
        assert np.array_equal(host(got).view(np.uint32), host(fresh).view(np.uint32)), n
        want = _oracle(q, k[:, :, :n], v[:, :, :n])
        assert max_abs(host(got), want) <= TOL, (n, max_abs(host(got), want))


@pytest.mark.parametrize("hq,hkv,r,causal", [(32, 8, 1, False), (16, 2, 2, True)])
def test_mfma8_fused_window(hq, hkv, r, causal):
    """N packed 8-bit tokens plus a 48-token float32 window: the fused form
    (window partial + matrix-core attend and combine) against the oracle and
    against the general-kernel form."""
    B, n, win, D = 2, 2000, 48, 128
    wl = Workload("win8", B, hq, hkv, r, n + win, D, ((BITS, GROUP),))
    q, k, v = make_qkv(wl, 26)
    announce(f"mfma 8-bit fused window hq={hq} hkv={hkv} R={r} causal={causal}")
    want = O.attend_window(q, k, v, win, BITS, GROUP, causal=causal)
    kc, ks = kvq.pack_k(dev(k[:, :, :n]), BITS, GROUP)
    vc, vs = kvq.pack_v(dev(v[:, :, :n]), BITS, GROUP)
    kw, vw, qd = dev(k[:, :, n:]), dev(v[:, :, n:]), dev(q)
    for splits in (1, 3, 0):
        fused = host(kvq.attend_window(qd, kc, ks, vc, vs, kw, vw, n, BITS, GROUP,
                                       num_splits=splits, causal=causal))
        assert max_abs(fused, want) <= TOL, (splits, max_abs(fused, want))
        if splits:
            small = kvq.new_workspace(B, hq, hkv, r, n + win, D, splits)
            general = host(kvq.attend_window(qd, kc, ks, vc, vs, kw, vw, n, BITS, GROUP,
                                             num_splits=splits, workspace=small, causal=causal))
            assert max_abs(fused, general) <= SPLIT_TOL, splits


def test_mfma8_gqa_n4096_full():
    """The 8 sequences x 4096 tokens, GQA 32/8 cache in 8-bit group 32 (the
    shape bench.py times for this format): every output against the oracle."""
    w = WORKLOADS["gqa_n4096"]
    q, k, v = make_qkv(w, 0)
    announce("mfma 8-bit gqa_n4096 full")
    want = _oracle(q, k, v)
    cache = _cache(k, v)
    outs = {}
    for splits in (1, 16, 0):
        outs[splits] = host(kvq.attend(dev(q), *cache, w.N, BITS, GROUP, num_splits=splits,
                                       variant="mfma"))
        assert max_abs(outs[splits], want) <= TOL, (splits, max_abs(outs[splits], want))
    assert max_abs(outs[1], outs[0]) <= SPLIT_TOL
