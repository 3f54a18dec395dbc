"""GPU parity of the mixed cache (kvq_attend_window): N packed tokens plus the
W most recent in float32, against the oracle's attend_window (<= 1e-4),
including the causal chunk, an empty packed part, and a decode loop that
moves the window's oldest token into a growing packed cache."""
import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import Workload, make_qkv

from gpu_helpers import announce, dev, host, max_abs

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")

TOL = 1e-4


@pytest.mark.parametrize("B,hq,hkv,r,n,w,d,bits,group,causal", [
    (2, 8, 2, 1, 500, 16, 128, 4, 32, False),
    (1, 4, 1, 4, 1021, 64, 32, 4, 8, False),
    (1, 2, 2, 8, 300, 33, 64, 8, 8, True),
    (2, 4, 2, 4, 0, 40, 128, 4, 32, False),     # no packed token at all
    (1, 2, 1, 2, 4096, 1, 128, 4, 32, True),
    # 8 KV heads (the 4-row kernel places window parts after every head's
    # packed splits) with four window parts, 8-bit and 4-bit
    (1, 32, 8, 1, 700, 100, 128, 8, 32, False),
    (3, 24, 8, 1, 1500, 97, 128, 4, 32, True),
])
def test_attend_window(B, hq, hkv, r, n, w, d, bits, group, causal):
    wl = Workload("win", B, hq, hkv, r, n + w, d, ((bits, group),))
    q, k, v = make_qkv(wl, 9)
    announce(f"attend_window B={B} hq={hq} hkv={hkv} R={r} N={n} W={w} D={d} {bits}b g{group} "
             f"causal={causal}")
    want = O.attend_window(q, k, v, w, bits, group, causal=causal)
    cap = max(n, 1)
    kp = np.zeros((B, hkv, cap, d), np.float32)
    vp = np.zeros((B, hkv, cap, d), np.float32)
    kp[:, :, :n], vp[:, :, :n] = k[:, :, :n], v[:, :, :n]
    kc, ks = kvq.pack_k(dev(kp), bits, group)
    vc, vs = kvq.pack_v(dev(vp), bits, group)
    kw, vw = dev(k[:, :, n:]), dev(v[:, :, n:])
    for splits in (1, 3, 0):
        got = host(kvq.attend_window(dev(q), kc, ks, vc, vs, kw, vw, n, bits, group,
                                     capacity=cap, num_splits=splits, causal=causal))
        assert np.isfinite(got).all()
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


@pytest.mark.parametrize("hq,hkv,r,causal", [(32, 8, 1, False), (16, 2, 2, True), (8, 8, 4, True),
                                             (8, 1, 1, False), (4, 2, 4, True)])
def test_fused_window_equals_general_kernel(hq, hkv, r, causal):
    """The fused form (window partials + matrix-core combine; the 48-token
    window in two parts, or in one when the workspace has a single extra
    slot) against the general kernel on the same call (a workspace with no
    extra slot forces the latter), and all against the oracle."""
    B, n, w, D = 2, 2000, 48, 128
    wl = Workload("fused", B, hq, hkv, r, n + w, D, ((4, 32),))
    q, k, v = make_qkv(wl, 13)
    announce(f"window fused vs general hq={hq} hkv={hkv} R={r} causal={causal}")
    want = O.attend_window(q, k, v, w, 4, 32, causal=causal)
    kc, ks = kvq.pack_k(dev(k[:, :, :n]), 4, 32)
    vc, vs = kvq.pack_v(dev(v[:, :, :n]), 4, 32)
    kw, vw, qd = dev(k[:, :, n:]), dev(v[:, :, n:]), dev(q)
    for splits in (1, 3, 0):
        fused = host(kvq.attend_window(qd, kc, ks, vc, vs, kw, vw, n, 4, 32, num_splits=splits,
                                       causal=causal))
        assert max_abs(fused, want) <= TOL, (splits, max_abs(fused, want))
        if splits:  # exactly `splits` slots: no room for the window's, so the general kernel runs
            small = kvq.new_workspace(B, hq, hkv, r, n + w, D, splits)
            general = host(kvq.attend_window(qd, kc, ks, vc, vs, kw, vw, n, 4, 32,
                                             num_splits=splits, workspace=small, causal=causal))
            assert max_abs(fused, general) <= 2e-5, splits
            assert max_abs(general, want) <= TOL, splits
            # one slot more: the fused form with the whole window in one part
            # (the default workspace has one per 32 window tokens, here 2)
            one = kvq.new_workspace(B, hq, hkv, r, n + w, D, splits + 1)
            fused1 = host(kvq.attend_window(qd, kc, ks, vc, vs, kw, vw, n, 4, 32,
                                            num_splits=splits, workspace=one, causal=causal))
            assert max_abs(fused1, fused) <= 2e-5, splits
            assert max_abs(fused1, want) <= TOL, splits


def test_decode_loop_with_window():
    """Each step: the new token joins the float32 window; once it holds W
    tokens the oldest moves into the packed cache (kvq_append)."""
    B, hq, hkv, d, cap, W = 1, 4, 2, 128, 160, 8
    wl = Workload("loop", B, hq, hkv, 1, cap + W, d, ((4, 32),))
    q, k, v = make_qkv(wl, 10)
    announce("decode loop with an 8-token window")
    cache = kvq.new_cache(B, hkv, cap, d, 4, 32)
    kd, vd, qd = dev(k), dev(v), dev(q)
    n_packed = 0
    for t in range(1, 150):                      # t tokens so far
        w = min(t, W)
        if t > W:                                # token t - W - 1 leaves the window
            j = t - W - 1
            kvq.append(kd[:, :, j:j + 1].contiguous(), vd[:, :, j:j + 1].contiguous(), n_packed,
                       cache, cap, 4, 32)
            n_packed += 1
        if t % 37 == 0 or t in (1, 8, 9, 149):
            got = host(kvq.attend_window(qd, *cache[:4], kd[:, :, t - w:t].contiguous(),
                                         vd[:, :, t - w:t].contiguous(), n_packed, 4, 32,
                                         capacity=cap))
            want = O.attend_window(q, k[:, :, :t], v[:, :, :t], w, 4, 32)
            assert max_abs(got, want) <= TOL, (t, max_abs(got, want))


def test_window_full_size_sampled():
    """The 8 x 4096-token mixed cache bench.py times (the last 64 tokens float32),
    sampled KV heads against the oracle."""
    from workloads import WORKLOADS
    w = WORKLOADS["gqa_n4096"]
    q, k, v = make_qkv(w, 12)
    win = 64
    npk = w.N - win
    announce("window full size gqa_n4096 W=64")
    kc, ks = kvq.pack_k(dev(k[:, :, :npk]), 4, 32)
    vc, vs = kvq.pack_v(dev(v[:, :, :npk]), 4, 32)
    got = host(kvq.attend_window(dev(q), kc, ks, vc, vs, dev(k[:, :, npk:]), dev(v[:, :, npk:]),
                                 npk, 4, 32))
    rep = w.Hq // w.Hkv
    for b, h in ((0, 0), (3, 5), (7, 7)):
        qs = q[b:b + 1, h * rep:(h + 1) * rep]
        want = O.attend_window(qs, k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], win, 4, 32)
        assert max_abs(got[b:b + 1, h * rep:(h + 1) * rep], want) <= TOL, (b, h)


@pytest.mark.parametrize("bits,group", [(4, 8), (8, 16), (4, 64)], ids=["4b-g8", "8b-g16", "4b-g64"])
@pytest.mark.parametrize("hq,hkv,r,causal", [(32, 8, 1, False), (16, 2, 2, True), (8, 8, 1, True),
                                             (4, 1, 2, False)])
def test_fused_window_on_the_streaming_kernel(bits, group, hq, hkv, r, causal):
    """Mixed caches in the formats the streaming kernel takes: its launch with
    window parts after the packed splits, against the oracle and against the
    general kernel on the same call (a workspace with no extra slot forces
    the latter)."""
    B, n, w, D = 2, 1500, 70, 128
    wl = Workload("stream_win", B, hq, hkv, r, n + w, D, ((bits, group),))
    q, k, v = make_qkv(wl, 17)
    announce(f"window on the streaming kernel hq={hq} hkv={hkv} R={r} {bits}b g{group} "
             f"causal={causal}")
    want = O.attend_window(q, k, v, w, bits, group, causal=causal)
    kc, ks = kvq.pack_k(dev(k[:, :, :n]), bits, group)
    vc, vs = kvq.pack_v(dev(v[:, :, :n]), bits, group)
    kw, vw, qd = dev(k[:, :, n:]), dev(v[:, :, n:]), dev(q)
    for splits in (1, 3, 0):
        fused = host(kvq.attend_window(qd, kc, ks, vc, vs, kw, vw, n, bits, group,
                                       num_splits=splits, causal=causal))
        assert np.isfinite(fused).all(), splits
        assert max_abs(fused, want) <= TOL, (splits, max_abs(fused, want))
        if splits:
            small = kvq.new_workspace(B, hq, hkv, r, n + w, D, splits)
            general = host(kvq.attend_window(qd, kc, ks, vc, vs, kw, vw, n, bits, group,
                                             num_splits=splits, workspace=small, causal=causal))
            assert max_abs(fused, general) <= 2e-5, (splits, max_abs(fused, general))
