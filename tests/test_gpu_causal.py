"""GPU parity of the causal chunk (kvq_attend_cache with KVQ_ATTEND_CAUSAL):
the R queries of each head are the last R positions, query r reads tokens
j <= N - R + r.  Against the float64 oracle (<= 1e-4), across split counts
(many splits see no legal key for some rows), with rows that have no legal
key at all (zeros), and on a cache grown by appends."""
import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import Workload, make_qkv

from gpu_helpers import announce, dev, host, max_abs, oracle_pack

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")

TOL = 1e-4


MFMA_OK = {(4, 32, 128), (8, 32, 128)}   # (bits, group, D) the matrix-core kernels take (<= 32 rows)


@pytest.mark.parametrize("variant", ["valu", "mfma", "auto"])
@pytest.mark.parametrize("B,hq,hkv,r,n,d,bits,group", [
    (2, 8, 2, 4, 100, 128, 4, 32),      # 16 rows per KV head: 32-row kernel
    (1, 4, 1, 8, 5, 64, 8, 8),          # N < R: queries 0..2 have no legal key
    (2, 4, 4, 3, 1021, 32, 4, 8),
    (1, 2, 1, 16, 40, 128, 4, 32),      # 32 rows per KV head
    (1, 8, 8, 2, 4097, 128, 4, 32),     # 2 rows: 4-row kernel
    (1, 2, 2, 4, 3, 128, 4, 32),        # 4-row kernel, N < R
    (2, 4, 1, 8, 70, 128, 4, 32),       # 32 rows, the mask spans two 32-token blocks
    (1, 4, 2, 2, 33, 128, 4, 32),       # 4 rows, tokens 32.. in a second block
    (2, 4, 1, 2, 70, 128, 4, 32),       # 8 rows per KV head
])
def test_causal_chunk(B, hq, hkv, r, n, d, bits, group, variant):
    if variant == "mfma" and (bits, group, d) not in MFMA_OK:
        pytest.skip("outside the matrix-core kernels' format")
    w = Workload("causal", B, hq, hkv, r, n, d, ((bits, group),))
    q, k, v = make_qkv(w, 5)
    announce(f"causal B={B} hq={hq} hkv={hkv} R={r} N={n} D={d} {bits}b g{group} {variant}")
    kc, ks, vc, vs = oracle_pack(k, v, bits, group)
    want = O.attend_packed(q, kc, ks, vc, vs, n, bits, group, causal=True)
    gk, gks = kvq.pack_k(dev(k), bits, group)
    gv, gvs = kvq.pack_v(dev(v), bits, group)
    qd = dev(q)
    empty = O.causal_mask(n, r).sum(axis=1) == 0          # queries with no legal key
    for splits in (1, 3, 0, 64):
        got = host(kvq.attend(qd, gk, gks, gv, gvs, n, bits, group, num_splits=splits,
                              variant=variant, causal=True))
        assert np.isfinite(got).all(), splits
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))
        assert (got[:, :, empty] == 0).all()


@pytest.mark.parametrize("hq,hkv,r", [(8, 2, 2), (8, 1, 4)])
def test_causal_matrix_core_equals_general_kernel(hq, hkv, r):
    """Both kernel families on one causal problem agree within the split
    tolerance (a different summation order only)."""
    w = Workload("causal_x", 2, hq, hkv, r, 1500, 128, ((4, 32),))
    q, k, v = make_qkv(w, 8)
    announce(f"causal mfma vs valu hq={hq} hkv={hkv} R={r}")
    gk, gks = kvq.pack_k(dev(k), 4, 32)
    gv, gvs = kvq.pack_v(dev(v), 4, 32)
    qd = dev(q)
    a = host(kvq.attend(qd, gk, gks, gv, gvs, w.N, 4, 32, variant="mfma", causal=True))
    b = host(kvq.attend(qd, gk, gks, gv, gvs, w.N, 4, 32, variant="valu", causal=True))
    assert max_abs(a, b) <= 2e-5


def test_single_query_causal_is_the_unmasked_call():
    w = Workload("causal1", 2, 8, 2, 1, 777, 128, ((4, 32),))
    q, k, v = make_qkv(w, 6)
    announce("causal R=1 on the matrix-core kernel")
    gk, gks = kvq.pack_k(dev(k), 4, 32)
    gv, gvs = kvq.pack_v(dev(v), 4, 32)
    qd = dev(q)
    a = host(kvq.attend(qd, gk, gks, gv, gvs, w.N, 4, 32, variant="mfma", causal=True))
    b = host(kvq.attend(qd, gk, gks, gv, gvs, w.N, 4, 32, variant="mfma"))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_multi_token_step_on_a_growing_cache():
    """Append R tokens, then attend them causally (a multi-token decode step)."""
    B, hq, hkv, r, D, cap = 2, 8, 2, 4, 128, 300
    w = Workload("grow", B, hq, hkv, r, cap, D, ((4, 32),))
    q, k, v = make_qkv(w, 7)
    announce("causal multi-token steps on a growing cache")
    cache = kvq.new_cache(B, hkv, cap, D, 4, 32)
    kd, vd, qd = dev(k), dev(v), dev(q)
    n = 0
    for t in (200, r, r, r, 1, r):
        kvq.append(kd[:, :, n:n + t].contiguous(), vd[:, :, n:n + t].contiguous(), n, cache,
                   cap, 4, 32)
        n += t
        got = host(kvq.attend(qd, *cache[:4], n, 4, 32, capacity=cap, causal=True))
        kc, ks, vc, vs = oracle_pack(k[:, :, :n], v[:, :, :n], 4, 32)
        want = O.attend_packed(q, kc, ks, vc, vs, n, 4, 32, causal=True)
        assert max_abs(got, want) <= TOL, (n, max_abs(got, want))


@pytest.mark.parametrize("name,r,splits", [("gqa_n4096", 4, 0), ("gqa_n32768", 4, 16)])
def test_causal_full_size_sampled(name, r, splits):
    """The full-size caches with a causal chunk of R queries per head (the
    shapes bench.py times for the causal step), on the matrix-core kernels;
    the oracle recomputes sampled KV heads."""
    import dataclasses
    from workloads import WORKLOADS
    w = dataclasses.replace(WORKLOADS[name], R=r)
    q, k, v = make_qkv(w, 11)
    announce(f"causal full size {name} R={r} splits={splits}")
    gk, gks = kvq.pack_k(dev(k), 4, 32)
    gv, gvs = kvq.pack_v(dev(v), 4, 32)
    got = host(kvq.attend(dev(q), gk, gks, gv, gvs, w.N, 4, 32, num_splits=splits,
                          variant="mfma", causal=True))
    rep = w.Hq // w.Hkv
    for b, h in ((0, 0), (w.B - 1, w.Hkv - 1)):
        qs = q[b:b + 1, h * rep:(h + 1) * rep]
        kc, ks, vc, vs = oracle_pack(k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], 4, 32)
        want = O.attend_packed(qs, kc, ks, vc, vs, w.N, 4, 32, causal=True)
        assert max_abs(got[b:b + 1, h * rep:(h + 1) * rep], want) <= TOL, (b, h)
