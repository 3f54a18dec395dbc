"""GPU parity of kvq_pack and kvq_dequant: bit-exact against the oracle."""
import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import WORKLOADS, make_crafted, make_qkv

from gpu_helpers import announce, dev, host, oracle_pack, oracle_store

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")


def _check_pack_dequant(k, v, bits, group, label):
    announce(f"pack/dequant {label} shape={k.shape} bits={bits} group={group}")
    kc, ks, vc, vs = oracle_pack(k, v, bits, group)
    skc, sks, svc, svs = oracle_store(k, v, bits, group)
    gkc, gks = kvq.pack_k(dev(k), bits, group)
    gvc, gvs = kvq.pack_v(dev(v), bits, group)
    assert np.array_equal(host(gkc), skc)
    assert np.array_equal(host(gks).view(np.uint32), sks.view(np.uint32))
    assert np.array_equal(host(gvc), svc)
    assert np.array_equal(host(gvs).view(np.uint32), svs.view(np.uint32))
    B, H, N, D = k.shape
    kd = host(kvq.dequant_k(gkc, gks, N, D, bits, group))
    vd = host(kvq.dequant_v(gvc, gvs, N, D, bits, group))
    assert np.array_equal(kd.view(np.uint32), O.dequant_k(kc, ks, k.shape, bits, group).view(np.uint32))
    assert np.array_equal(vd.view(np.uint32), O.dequant_v(vc, vs, v.shape, bits, group).view(np.uint32))


@pytest.mark.parametrize("name,bits,group,dist", [
    ("single_n128", 4, 32, "clean"),
    ("single_n512", 4, 8, "clean"), ("single_n512", 4, 32, "clean"),
    ("single_n512", 8, 8, "clean"), ("single_n512", 8, 32, "clean"),
    ("single_n1024", 4, 8, "clean"), ("single_n1024", 4, 8, "early"),
    ("single_n1024", 4, 8, "late"),
    ("gqa_n4096", 4, 32, "clean"),
])
def test_pack_bit_exact_workloads(name, bits, group, dist):
    _, k, v = make_qkv(WORKLOADS[name], 0, dist)
    _check_pack_dequant(k, v, bits, group, f"{name}/{dist}")


@pytest.mark.parametrize("bits,group", [(4, 8), (4, 32), (8, 8), (8, 32), (4, 2), (8, 6)])
def test_pack_ragged_35x13(bits, group):
    x = make_crafted("ragged")
    k = np.stack([x, 2 * x])[None]         # [1, 2, 35, 13]
    v = np.stack([-x, x * 0.5])[None]
    _check_pack_dequant(k, v, bits, group, "ragged35x13")


@pytest.mark.parametrize("kind", ["zeros", "ties", "tiny"])
@pytest.mark.parametrize("bits", [4, 8])
def test_pack_crafted(kind, bits):
    x = make_crafted(kind)
    k = x[None, None]
    _check_pack_dequant(k, k.copy(), bits, 8 if kind == "ties" else 32, kind)


@pytest.mark.parametrize("N,D,bits,group", [
    (100, 300, 4, 32),   # D above the LDS-staged limit: two-pass kernels
    (77, 256, 4, 64),    # K groups longer than a block: scale pass + staged codes
    (65, 40, 8, 16),     # two K groups per block, staged scales and codes
    (33, 8, 4, 2),       # sixteen K groups per block, tiny head dim
    (50, 24, 4, 6),      # group not dividing the block: scale pass + staged codes
])
def test_pack_kernel_paths(N, D, bits, group):
    """Every packing path (LDS-staged per block, with local or precomputed K
    scales, and the two-pass fallback) against the oracle, ragged N."""
    rng = np.random.default_rng(N * 1000 + D)
    k = rng.standard_normal((2, 2, N, D), dtype=np.float32) * np.float32(2.0)
    v = rng.standard_normal((2, 2, N, D), dtype=np.float32)
    k[0, 1, : min(N, 20)] = 0.0
    _check_pack_dequant(k, v, bits, group, f"paths N={N} D={D}")


def test_pack_multi_head_random():
    rng = np.random.default_rng(77)
    k = (rng.standard_normal((3, 5, 333, 64), dtype=np.float32) * np.float32(3.0))
    v = rng.standard_normal((3, 5, 333, 64), dtype=np.float32)
    k[1, 2, :40] = 0.0
    _check_pack_dequant(k, v, 4, 32, "multihead")


def test_pack_full_gqa_n32768_sampled_heads():
    """Full-size workload: GPU packs the whole cache; sampled (b, h) heads are
    compared byte for byte with the oracle's packing of the same heads."""
    w = WORKLOADS["gqa_n32768"]
    announce("pack gqa_n32768 full, sampled heads")
    _, k, v = make_qkv(w, 0)
    gkc, gks = kvq.pack_k(dev(k), 4, 32)
    gvc, gvs = kvq.pack_v(dev(v), 4, 32)
    for b, h in ((0, 0), (7, 3), (15, 7)):
        kc, ks, vc, vs = oracle_store(k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], 4, 32)
        assert np.array_equal(host(gkc[b:b + 1, h:h + 1]), kc)
        assert np.array_equal(host(gks[b:b + 1, h:h + 1]), ks)
        assert np.array_equal(host(gvc[b:b + 1, h:h + 1]), vc)
        assert np.array_equal(host(gvs[b:b + 1, h:h + 1]), vs)


@pytest.mark.parametrize("D", [8, 6])    # four-feature and one-element dequant kernels
def test_pack_dequant_more_heads_than_a_grid_row(D):
    """66,000 (batch, head) pairs, more than one grid dimension holds: the
    dequant grid spreads heads over two dimensions; every byte and float
    against the oracle."""
    rng = np.random.default_rng(90 + D)
    k = rng.standard_normal((1100, 60, 3, D), dtype=np.float32)
    v = rng.standard_normal((1100, 60, 3, D), dtype=np.float32)
    _check_pack_dequant(k, v, 4, 2, f"heads=66000 D={D}")
