"""GPU parity of kvq_attend (and the decode-all baseline) against the float64
oracle on the same quantized cache: max abs error <= 1e-4."""
import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import WORKLOADS, Workload, make_qkv

from gpu_helpers import announce, dev, host, max_abs, oracle_pack

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")

TOL = 1e-4          # max abs error vs the float64 oracle (unit-variance inputs)
SPLIT_TOL = 2e-5    # between split counts / kernels on the GPU


def _gpu_cache(k, v, bits, group):
    gkc, gks = kvq.pack_k(dev(k), bits, group)
    gvc, gvs = kvq.pack_v(dev(v), bits, group)
    return gkc, gks, gvc, gvs


def _run(q, cache, n, bits, group, **kw):
    return host(kvq.attend(dev(q), *cache, n, bits, group, **kw))


def _oracle(q, k, v, bits, group):
    kc, ks, vc, vs = oracle_pack(k, v, bits, group)
    return O.attend_packed(q, kc, ks, vc, vs, k.shape[2], bits, group)


VARIANTS = ["valu"]                 # head dim 32: VALU kernel only
MFMA_VARIANTS = ["valu", "mfma", "auto"]  # 4-bit g32 D=128 with <= 32 rows per KV head


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("name,bits,group,dist", [
    ("single_n128", 4, 32, "clean"),
    ("single_n512", 4, 8, "clean"), ("single_n512", 4, 32, "clean"),
    ("single_n512", 8, 8, "clean"), ("single_n512", 8, 32, "clean"),
    ("single_n1024", 4, 8, "clean"), ("single_n1024", 4, 8, "early"),
    ("single_n1024", 4, 8, "late"),
])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attend_small_workloads(name, bits, group, dist, seed, variant):
    w = WORKLOADS[name]
    q, k, v = make_qkv(w, seed, dist)
    announce(f"attend {name}/{dist} seed={seed} {bits}b g{group} {variant}")
    want = _oracle(q, k, v, bits, group)
    cache = _gpu_cache(k, v, bits, group)
    for splits in (1, 2, 0):
        got = _run(q, cache, w.N, bits, group, num_splits=splits, variant=variant)
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_float32_cache_and_decode_all(seed):
    """The float32-cache reference and decode-all (dequant + attend_f32)."""
    w = WORKLOADS["single_n512"]
    q, k, v = make_qkv(w, seed)
    announce(f"attend_f32 single_n512 seed={seed}")
    got = host(kvq.attend_f32(dev(q), dev(k), dev(v)))
    assert max_abs(got, O.attend_dense(q, k, v)) <= TOL
    for bits, group in w.formats:
        gkc, gks, gvc, gvs = _gpu_cache(k, v, bits, group)
        kd = kvq.dequant_k(gkc, gks, w.N, w.D, bits, group)
        vd = kvq.dequant_v(gvc, gvs, w.N, w.D, bits, group)
        got = host(kvq.attend_f32(dev(q), kd, vd, num_splits=3))
        assert max_abs(got, _oracle(q, k, v, bits, group)) <= TOL


@pytest.mark.parametrize("variant", MFMA_VARIANTS)
def test_attend_gqa_n4096_full(variant):
    w = WORKLOADS["gqa_n4096"]
    q, k, v = make_qkv(w, 0)
    announce(f"attend gqa_n4096 full {variant}")
    want = _oracle(q, k, v, 4, 32)
    cache = _gpu_cache(k, v, 4, 32)
    outs = {}
    for splits in (1, 2, 16, 0):
        outs[splits] = _run(q, cache, w.N, 4, 32, num_splits=splits, variant=variant)
        assert max_abs(outs[splits], want) <= TOL, (splits, max_abs(outs[splits], want))
    for s in (1, 2, 16):
        assert max_abs(outs[s], outs[0]) <= SPLIT_TOL


@pytest.mark.parametrize("variant", MFMA_VARIANTS)
@pytest.mark.parametrize("seed", [0, 1])
def test_attend_gqa_n32768_sampled(variant, seed):
    """Full-size long-context workload (16 splits).  The GPU attends over the
    whole cache; the oracle recomputes every query row of sampled KV heads."""
    w = WORKLOADS["gqa_n32768"]
    q, k, v = make_qkv(w, seed)
    announce(f"attend gqa_n32768 full seed={seed} {variant}")
    cache = _gpu_cache(k, v, 4, 32)
    got = _run(q, cache, w.N, 4, 32, num_splits=w.num_splits, variant=variant)
    # 64 splits: runs of 16 splits per workgroup, 4 whole splits per wave
    more = _run(q, cache, w.N, 4, 32, num_splits=64, variant=variant) if seed == 0 else None
    rep = w.Hq // w.Hkv
    for b, h in ((0, 0), (5, 6), (15, 7)):
        qs = q[b:b + 1, h * rep:(h + 1) * rep]
        want = _oracle(qs, k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], 4, 32)
        assert max_abs(got[b:b + 1, h * rep:(h + 1) * rep], want) <= TOL
        if more is not None:
            assert max_abs(more[b:b + 1, h * rep:(h + 1) * rep], want) <= TOL
    if more is not None:
        assert max_abs(more, got) <= SPLIT_TOL


def test_attend_gqa_n32768_8bit_sampled():
    """The long-context workload in 8-bit group 32 at its 16 splits (4 splits
    per workgroup, two row tiles): sampled KV heads against the oracle."""
    w = WORKLOADS["gqa_n32768"]
    q, k, v = make_qkv(w, 2)
    announce("attend gqa_n32768 8-bit full")
    cache = _gpu_cache(k, v, 8, 32)
    got = _run(q, cache, w.N, 8, 32, num_splits=w.num_splits)
    rep = w.Hq // w.Hkv
    for b, h in ((0, 0), (9, 3), (15, 7)):
        qs = q[b:b + 1, h * rep:(h + 1) * rep]
        want = _oracle(qs, k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], 8, 32)
        assert max_abs(got[b:b + 1, h * rep:(h + 1) * rep], want) <= TOL


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("n", [1, 7, 35, 1021, 4097])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_attend_ragged_tokens(n, d, variant):
    w = Workload("ragged", 2, 8, 2, 2, n, d, ((4, 32),))
    q, k, v = make_qkv(w, 3)
    announce(f"attend ragged n={n} d={d} {variant}")
    want = _oracle(q, k, v, 4, 32)
    cache = _gpu_cache(k, v, 4, 32)
    for splits in (1, 3, 0, 64):
        got = _run(q, cache, n, 4, 32, num_splits=splits, variant=variant)
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


def test_attend_sm_scale_and_peaky_scores():
    """Explicit temperature, and large scores that need the max shift."""
    w = WORKLOADS["single_n512"]
    q, k, v = make_qkv(w, 2)
    announce("attend sm_scale")
    cache = _gpu_cache(k, v, 4, 32)
    kc, ks, vc, vs = oracle_pack(k, v, 4, 32)
    for sm in (0.05, 1.0, 3.0):
        got = _run(q, cache, w.N, 4, 32, sm_scale=sm, num_splits=4)
        want = O.attend_packed(q, kc, ks, vc, vs, w.N, 4, 32, sm_scale=sm)
        assert np.all(np.isfinite(got))
        assert max_abs(got, want) <= TOL


def _counters(ws, B, Hkv):
    """The arrival counters: one per (batch, KV head), 256 bytes apart, at the
    start of the workspace."""
    return host(ws)[:256 * B * Hkv]


@pytest.mark.parametrize("variant", MFMA_VARIANTS)
def test_attend_deterministic_and_counters_reset(variant):
    w = WORKLOADS["gqa_n4096"]
    q, k, v = make_qkv(w, 1)
    announce(f"attend determinism {variant}")
    cache = _gpu_cache(k, v, 4, 32)
    ws = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D, 0)
    a = _run(q, cache, w.N, 4, 32, workspace=ws, variant=variant)
    b = _run(q, cache, w.N, 4, 32, workspace=ws, variant=variant)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert not _counters(ws, w.B, w.Hkv).any()  # every call leaves the counters at zero


def test_attend_variants_share_one_workspace():
    """Split paths of every kernel, one after another on one workspace with
    different split counts and row shapes: the arrival counters sit where the
    (batch, KV head) count alone puts them, and each call leaves them zero."""
    w = WORKLOADS["gqa_n4096"]
    q, k, v = make_qkv(w, 2)
    announce("attend shared workspace")
    want = _oracle(q, k, v, 4, 32)
    cache = _gpu_cache(k, v, 4, 32)
    ws = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D, 16)
    for variant, splits in (("valu", 16), ("mfma", 16), ("valu", 3), ("mfma", 5), ("mfma", 0),
                            ("auto", 0), ("valu", 0)):
        got = _run(q, cache, w.N, 4, 32, num_splits=splits, workspace=ws, variant=variant)
        assert max_abs(got, want) <= TOL, (variant, splits)
        assert not _counters(ws, w.B, w.Hkv).any(), (variant, splits)
    # 16 query rows per KV head (the 32-row matrix-core kernel), fewer heads:
    # their counters are a prefix of the zero counters above
    w2 = Workload("ws32", 2, 16, 2, 2, 1021, 128, ((4, 32),))
    q2, k2, v2 = make_qkv(w2, 3)
    want2 = _oracle(q2, k2, v2, 4, 32)
    cache2 = _gpu_cache(k2, v2, 4, 32)
    for variant, splits in (("mfma", 7), ("valu", 16), ("mfma", 16), ("auto", 0)):
        got = _run(q2, cache2, w2.N, 4, 32, num_splits=splits, workspace=ws, variant=variant)
        assert max_abs(got, want2) <= TOL, (variant, splits)
        assert not _counters(ws, w2.B, w2.Hkv).any(), (variant, splits)


@pytest.mark.parametrize("variant,shape,splits", [
    ("mfma", (8, 32, 8, 1, 4096), 0), ("mfma", (2, 16, 2, 2, 1021), 7),
    ("valu", (8, 32, 8, 1, 4096), 0)])
def test_attend_graph_replay(variant, shape, splits):
    """Calls captured in a HIP graph (two per graph, sharing one workspace, as
    a serving loop or the timed bench steps would launch them) give the eager
    result bit for bit on every replay, with eager work and host syncs in
    between; the split counters stay reset."""
    import torch
    B, Hq, Hkv, R, N = shape
    w = Workload("graph", B, Hq, Hkv, R, N, 128, ((4, 32),))
    q, k, v = make_qkv(w, 4)
    announce(f"attend graph replay {variant} {shape} splits={splits}")
    cache = _gpu_cache(k, v, 4, 32)
    qd = dev(q)
    q2 = qd.flip(-1).contiguous()
    ws = kvq.new_workspace(B, Hq, Hkv, R, N, 128, splits)
    o1, o2 = torch.empty_like(qd), torch.empty_like(qd)

    def calls():
        kvq.attend(qd, *cache, N, 4, 32, num_splits=splits, workspace=ws, out=o1, variant=variant)
        kvq.attend(q2, *cache, N, 4, 32, num_splits=splits, workspace=ws, out=o2, variant=variant)
    calls()
    torch.cuda.synchronize()
    e1, e2 = o1.clone(), o2.clone()
    assert max_abs(host(e1), _oracle(q, k, v, 4, 32)) <= TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        o1.fill_(float("nan"))
        o2.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o1, e1) and torch.equal(o2, e2), rep
        assert not _counters(ws, B, Hkv).any(), rep
        kvq.attend(q2, *cache, N, 4, 32, num_splits=splits, workspace=ws, out=o1, variant=variant)
        torch.cuda.synchronize()


@pytest.mark.parametrize("hq,hkv,r", [(8, 2, 1), (2, 2, 3), (1, 1, 1), (4, 1, 1), (6, 3, 2)])
@pytest.mark.parametrize("n", [1, 7, 35, 1021, 4097])
def test_attend_mfma_ragged_and_gqa_shapes(hq, hkv, r, n):
    """Matrix-core kernel: 1..4 query rows per KV head, ragged token counts,
    empty trailing splits."""
    w = Workload("mfma", 2, hq, hkv, r, n, 128, ((4, 32),))
    q, k, v = make_qkv(w, 4)
    announce(f"attend mfma hq={hq} hkv={hkv} r={r} n={n}")
    want = _oracle(q, k, v, 4, 32)
    cache = _gpu_cache(k, v, 4, 32)
    for splits in (1, 3, 0, 64):
        got = _run(q, cache, n, 4, 32, num_splits=splits, variant="mfma")
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("hq,hkv,r", [(8, 1, 1), (5, 1, 1), (6, 3, 4), (7, 1, 1), (4, 1, 2)])
@pytest.mark.parametrize("n", [1, 35, 1021, 4097])
def test_attend_mfma_five_to_eight_rows(hq, hkv, r, n, bits):
    """5..8 query rows per KV head (a GQA group of 8 with one query, or 4
    heads x 2 queries) on the matrix-core path, ragged token counts, against
    the oracle and the general kernel."""
    w = Workload("rg2", 2, hq, hkv, r, n, 128, ((bits, 32),))
    q, k, v = make_qkv(w, 9)
    announce(f"attend mfma 5-8 rows hq={hq} hkv={hkv} r={r} n={n} {bits}b")
    want = _oracle(q, k, v, bits, 32)
    cache = _gpu_cache(k, v, bits, 32)
    general = _run(q, cache, n, bits, 32, num_splits=3, variant="valu")
    for splits in (1, 3, 0, 64):
        got = _run(q, cache, n, bits, 32, num_splits=splits, variant="mfma")
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))
        assert max_abs(got, general) <= SPLIT_TOL, (splits, max_abs(got, general))


@pytest.mark.parametrize("dist", ["clean", "early", "late"])
@pytest.mark.parametrize("scale_k", [False, True])
def test_attend_mfma_peaky_and_channel_scaled(dist, scale_k):
    """Biased keys (+4 sigma on 16 tokens) and log-uniform K channel scales
    concentrate the softmax: the hi/lo fp16 split must hold 1e-4 there."""
    w = Workload("peaky", 4, 16, 4, 1, 4096, 128, ((4, 32),), k_channel_scale=scale_k)
    q, k, v = make_qkv(w, 5, dist)
    announce(f"attend mfma peaky dist={dist} scale_k={scale_k}")
    want = _oracle(q, k, v, 4, 32)
    cache = _gpu_cache(k, v, 4, 32)
    for splits in (1, 0):
        got = _run(q, cache, w.N, 4, 32, num_splits=splits, variant="mfma")
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


def test_attend_mfma_rejects_unsupported():
    w = WORKLOADS["single_n128"]
    q, k, v = make_qkv(w, 0)
    cache = _gpu_cache(k, v, 4, 32)
    with pytest.raises(kvq.KvqError) as e:
        _run(q, cache, w.N, 4, 32, variant="mfma")
    assert e.value.status == kvq.KVQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("hq,hkv,r", [(8, 1, 4), (16, 2, 2), (5, 1, 1), (12, 3, 8), (6, 1, 3)])
@pytest.mark.parametrize("n", [1, 7, 35, 1021, 4097])
def test_attend_mfma32_ragged_and_gqa_shapes(hq, hkv, r, n):
    """32-row matrix-core kernel: 5..32 query rows per KV head (padded to 32),
    ragged token counts, empty trailing splits."""
    w = Workload("mfma32", 2, hq, hkv, r, n, 128, ((4, 32),))
    q, k, v = make_qkv(w, 6)
    announce(f"attend mfma32 hq={hq} hkv={hkv} r={r} n={n}")
    want = _oracle(q, k, v, 4, 32)
    cache = _gpu_cache(k, v, 4, 32)
    for splits in (1, 3, 0, 64):
        got = _run(q, cache, n, 4, 32, num_splits=splits, variant="mfma")
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


@pytest.mark.parametrize("dist", ["clean", "early", "late"])
@pytest.mark.parametrize("scale_k", [False, True])
def test_attend_mfma32_peaky_and_channel_scaled(dist, scale_k):
    """Heads shaped like the 32768-token workload (8 GQA heads x 4 queries per KV head), biased keys and
    log-uniform K channel scales."""
    w = Workload("peaky32", 2, 16, 2, 4, 4096, 128, ((4, 32),), k_channel_scale=scale_k)
    q, k, v = make_qkv(w, 7, dist)
    announce(f"attend mfma32 peaky dist={dist} scale_k={scale_k}")
    want = _oracle(q, k, v, 4, 32)
    cache = _gpu_cache(k, v, 4, 32)
    for splits in (1, 0):
        got = _run(q, cache, w.N, 4, 32, num_splits=splits, variant="mfma")
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


# (B, Hq, Hkv, R, N, bits, causal, splits).  Where KV heads x splits fill at
# least 4 rounds of 512 workgroups, each workgroup of the 32-row kernel takes
# a run of 4 ceil(heads x splits / 2048) consecutive splits, each wave
# attends whole splits of it, and the workgroup stores one partial for the
# run (a two-level combine).  The split counts leave a shorter last run
# (some waves without a split), splits past the last token hold no key, and
# the masked block is a split's first.
MULTI_SPLIT = [
    (2, 8, 1, 4, 5000, 4, False, 1001),     # 32 rows, runs of 4, last run 1
    (1, 12, 1, 1, 4097, 8, False, 2050),    # 8-bit, 12 rows, runs of 8 (2 per wave), last 2
    (3, 16, 2, 1, 3001, 4, False, 302),     # 8 rows, 6 heads, runs of 4, last run 2
    (2, 32, 1, 1, 100000, 4, False, 1030),  # 4 blocks per split, runs of 8, last run 6
    (64, 64, 8, 1, 256, 4, False, 4),       # 512 heads: one workgroup per head, a split per wave
    (1, 8, 1, 1, 4097, 4, False, 65535),    # the most splits: runs of 128 (32 per wave), last run 127
    (1, 32, 1, 1, 5000, 8, False, 2000),    # 8-bit, 32 rows (2 tiles), runs of 4
    # Causal (queries at N - R .. N - 1): the tokens past N - R masked for some
    # rows lie in one block or two; a wave attends its split's masked blocks
    # first.
    (2, 4, 1, 4, 2100, 4, True, 1201),      # one masked block, runs of 8
    (16, 16, 4, 8, 2084, 4, True, 40),      # 32 rows: blocks 64 and 65 masked, one split
    (16, 16, 4, 8, 2084, 4, True, 100),     # the two masked blocks in adjacent splits
    (16, 8, 2, 4, 2081, 4, True, 65),       # 16 rows (1 tile): two masked blocks, one split
    (16, 8, 2, 4, 2081, 8, True, 65),       # the same in 8-bit
    (16, 16, 4, 8, 2084, 8, True, 40),      # causal 8-bit 32 rows: one split per workgroup
    (64, 64, 8, 4, 2, 4, True, 4),          # N < R: queries with no legal key (output 0)
    (64, 64, 8, 4, 35, 4, True, 4),         # 512 heads, splits past the last token
]


@pytest.mark.parametrize("shape", MULTI_SPLIT,
                         ids=["B{}-Hq{}-Hkv{}-R{}-N{}-{}b-causal{}-s{}".format(*c)
                              for c in MULTI_SPLIT])
def test_attend_mfma32_several_splits_per_workgroup(shape):
    B, hq, hkv, r, n, bits, causal, splits = shape
    w = Workload("multi_split", B, hq, hkv, r, n, 128, ((bits, 32),))
    q, k, v = make_qkv(w, 9)
    announce(f"attend mfma32 several splits per workgroup {shape}")
    kc, ks, vc, vs = oracle_pack(k, v, bits, 32)
    want = O.attend_packed(q, kc, ks, vc, vs, n, bits, 32, causal=causal)
    cache = _gpu_cache(k, v, bits, 32)
    got = _run(q, cache, n, bits, 32, num_splits=splits, variant="mfma", causal=causal)
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= TOL, max_abs(got, want)
    if causal:
        empty = O.causal_mask(n, r).sum(axis=1) == 0
        assert (got[:, :, empty] == 0).all()
    one = _run(q, cache, n, bits, 32, num_splits=1, variant="mfma", causal=causal)
    assert max_abs(got, one) <= SPLIT_TOL


# 16 shapes drawn once (seeded) among those where the 32-row kernel takes
# several splits per workgroup: 4- and 8-bit, causal or not, 5..32 rows per
# KV head, ragged N up to 3000, split counts with uneven runs.
MULTI_SPLIT_DRAWN = [
    (8, 4, 2, 4, 2633, 4, True, 268), (8, 64, 8, 1, 2261, 4, False, 76),
    (4, 8, 2, 4, 185, 4, True, 397), (2, 32, 8, 2, 2487, 4, False, 374),
    (16, 8, 2, 2, 503, 8, True, 58), (8, 8, 4, 8, 2357, 8, False, 111),
    (3, 32, 4, 4, 1869, 4, False, 462), (16, 8, 8, 8, 1467, 4, False, 40),
    (4, 8, 1, 4, 2540, 8, False, 1053), (4, 8, 2, 2, 2771, 4, True, 214),
    (4, 4, 1, 2, 1402, 4, False, 412), (16, 4, 1, 8, 2145, 4, True, 143),
    (16, 2, 1, 4, 1058, 4, False, 292), (2, 8, 4, 4, 2585, 8, False, 376),
    (8, 8, 8, 8, 2137, 8, False, 85), (8, 8, 1, 2, 1148, 8, True, 259),
]


@pytest.mark.parametrize("shape", MULTI_SPLIT_DRAWN,
                         ids=["B{}-Hq{}-Hkv{}-R{}-N{}-{}b-causal{}-s{}".format(*c)
                              for c in MULTI_SPLIT_DRAWN])
def test_attend_mfma32_several_splits_drawn_shapes(shape):
    B, hq, hkv, r, n, bits, causal, splits = shape
    w = Workload("multi_drawn", B, hq, hkv, r, n, 128, ((bits, 32),))
    q, k, v = make_qkv(w, 10)
    announce(f"attend mfma32 drawn shape {shape}")
    kc, ks, vc, vs = oracle_pack(k, v, bits, 32)
    want = O.attend_packed(q, kc, ks, vc, vs, n, bits, 32, causal=causal)
    got = _run(q, _gpu_cache(k, v, bits, 32), n, bits, 32, num_splits=splits, variant="mfma",
               causal=causal)
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= TOL, max_abs(got, want)


@pytest.mark.parametrize("hq,r", [(4, 1), (16, 2)])
def test_attend_mfma_large_k_scales(hq, r):
    """K magnitudes large enough that K scales reach 32 (the 32-row kernel
    rescales such blocks by a power of two) and very peaky softmax."""
    w = Workload("bigk", 1, hq, 1, r, 1000, 128, ((4, 32),))
    q, k, v = make_qkv(w, 8)
    k = (k * np.float32(300.0)).astype(np.float32)
    k[0, 0, 500:532] *= np.float32(0.01)   # one group with small scales among large ones
    announce(f"attend mfma large K scales hq={hq} r={r}")
    want = _oracle(q, k, v, 4, 32)
    cache = _gpu_cache(k, v, 4, 32)
    for splits in (1, 0):
        got = _run(q, cache, w.N, 4, 32, num_splits=splits, variant="mfma")
        assert np.all(np.isfinite(got))
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))
