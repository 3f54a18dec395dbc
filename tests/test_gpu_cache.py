"""GPU parity of the growing cache: kvq_cache_clear + kvq_append are
bit-exact against the oracle's cache after n tokens (the packed prefix
zero-padded to the capacity) after every call, and kvq_attend_cache over the
first n tokens matches the float64 oracle (<= 1e-4) and, bit for bit, the
attention over a cache packed from those n tokens alone."""
import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import Workload, make_qkv

from gpu_helpers import announce, dev, host, max_abs, oracle_pack

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")

TOL = 1e-4


def _grow(k, v, cap, bits, group, chunks):
    """Append k, v [B,H,N,D] in the given chunk sizes; yield n after each call
    with the device cache."""
    import torch
    B, H, N, D = k.shape
    cache = kvq.new_cache(B, H, cap, D, bits, group)
    torch.cuda.synchronize()
    yield 0, cache
    n = 0
    kd, vd = dev(k), dev(v)
    for t in chunks:
        kvq.append(kd[:, :, n:n + t].contiguous(), vd[:, :, n:n + t].contiguous(), n, cache, cap,
                   bits, group)
        n += t
        torch.cuda.synchronize()
        yield n, cache


def _check_state(k, v, n, cap, bits, group, cache):
    want = O.cache_after(k, v, n, cap, bits, group)
    for name, got, w in zip(("k_codes", "k_scales", "v_codes", "v_scales"), cache[:4], want):
        g = host(got)
        assert g.shape == w.shape, name
        assert np.array_equal(g.view(np.uint8), w.view(np.uint8)), (name, n)
    # the tail holds the float32 K of the open group's tokens
    tail = host(cache[4])
    for t in range(n // group * group, n):
        assert np.array_equal(tail[:, :, t % group, :], k[:, :, t, :]), t


@pytest.mark.parametrize("bits,group,d,cap,chunks", [
    (4, 32, 128, 200, [1, 1, 30, 1, 32, 5, 64, 2, 31, 1]),
    (4, 8, 32, 100, [3, 5, 1, 8, 16, 7, 1, 1, 1, 40]),
    (8, 6, 24, 70, [1, 5, 6, 13, 2, 40]),
    (4, 64, 128, 150, [10, 60, 1, 70, 2]),        # K groups span two blocks
    (4, 2, 13, 35, [1, 2, 3, 29]),                # odd head dim, smallest group
    (8, 32, 40, 33, [33]),                        # the whole capacity in one call
])
def test_append_bit_exact_after_every_call(bits, group, d, cap, chunks):
    k = np.random.default_rng(0).standard_normal((2, 3, sum(chunks), d), dtype=np.float32)
    v = np.random.default_rng(1).standard_normal((2, 3, sum(chunks), d), dtype=np.float32)
    announce(f"append {bits}b g{group} d={d} cap={cap} chunks={chunks}")
    for n, cache in _grow(k, v, cap, bits, group, chunks):
        _check_state(k, v, n, cap, bits, group, cache)


def test_prompt_then_decode_steps():
    """A 1000-token prompt in one call, then single-token decode steps, at the
    matrix-core kernels' format."""
    B, H, D, cap = 2, 2, 128, 1100
    k = np.random.default_rng(2).standard_normal((B, H, 1040, D), dtype=np.float32)
    v = np.random.default_rng(3).standard_normal((B, H, 1040, D), dtype=np.float32)
    announce("append prompt 1000 then 40 decode steps")
    for n, cache in _grow(k, v, cap, 4, 32, [1000] + [1] * 40):
        if n in (0, 1000, 1001, 1023, 1024, 1025, 1040):
            _check_state(k, v, n, cap, 4, 32, cache)


@pytest.mark.parametrize("variant", ["mfma", "valu", "auto"])
@pytest.mark.parametrize("hq,hkv,r", [(8, 2, 1), (16, 2, 2)])   # 4 and 16 rows per KV head
def test_attend_cache_prefix(variant, hq, hkv, r):
    import torch
    cap, D = 1100, 128
    w = Workload("cache", 2, hq, hkv, r, cap, D, ((4, 32),))
    q, k, v = make_qkv(w, 4)
    announce(f"attend_cache {variant} rows={hq // hkv * r}")
    qd = dev(q)
    chunks = [1, 30, 2, 500, 488, 1]             # n = 1, 31, 33, 533, 1021, 1022
    for n, cache in _grow(k, v, cap, 4, 32, chunks):
        if n == 0:
            continue
        got = kvq.attend(qd, *cache[:4], n, 4, 32, variant=variant, capacity=cap)
        kc, ks, vc, vs = oracle_pack(k[:, :, :n], v[:, :, :n], 4, 32)
        want = O.attend_packed(q, kc, ks, vc, vs, n, 4, 32)
        assert max_abs(host(got), want) <= TOL, (n, max_abs(host(got), want))
        # the same call on a cache packed from the n tokens alone
        fk, fks = kvq.pack_k(dev(k[:, :, :n]), 4, 32)
        fv, fvs = kvq.pack_v(dev(v[:, :, :n]), 4, 32)
        fresh = kvq.attend(qd, fk, fks, fv, fvs, n, 4, 32, variant=variant)
        torch.cuda.synchronize()
        assert np.array_equal(host(got).view(np.uint32), host(fresh).view(np.uint32)), n
        for s in (1, 3):
            got_s = kvq.attend(qd, *cache[:4], n, 4, 32, num_splits=s, variant=variant,
                               capacity=cap)
            assert max_abs(host(got_s), want) <= TOL, (n, s)


@pytest.mark.parametrize("bits,group,d", [
    (4, 32, 128), (8, 32, 40), (8, 8, 24), (4, 8, 13), (4, 64, 128), (8, 64, 64), (4, 128, 32),
    (8, 6, 24),                                   # 6 per group: the general kernel
])
def test_single_token_appends_bit_exact(bits, group, d):
    """A run of one-token appends (the decode step's lane-parallel kernel
    where the group's byte count is a power of two <= 64), checked after
    every call, from an empty cache through several groups and blocks."""
    cap = 75
    k = np.random.default_rng(3).standard_normal((2, 3, cap, d), dtype=np.float32)
    v = np.random.default_rng(4).standard_normal((2, 3, cap, d), dtype=np.float32)
    announce(f"single-token appends {bits}b g{group} d={d}")
    for n, cache in _grow(k, v, cap, bits, group, [1] * cap):
        _check_state(k, v, n, cap, bits, group, cache)
