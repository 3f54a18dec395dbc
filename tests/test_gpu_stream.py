"""The streaming float32 kernel (KVQ_VARIANT_STREAM: 4- or 8-bit, groups 8 to
128, D = 128, up to 8 query rows per KV head) against the float64 oracle over
the same packed cache, max abs error <= 1e-4, and against the general
kernel; which kernel the automatic choice runs; what the variant rejects."""
import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import WORKLOADS, Workload, make_qkv

from gpu_helpers import announce, dev, host, max_abs, oracle_pack

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")
torch = pytest.importorskip("torch")

TOL = 1e-4        # vs the float64 oracle (unit-variance inputs)
KERNEL_TOL = 2e-5  # between kernels / split counts on the GPU


def _cache(k, v, bits, group):
    kc, ks = kvq.pack_k(dev(k), bits, group)
    vc, vs = kvq.pack_v(dev(v), bits, group)
    return kc, ks, vc, vs


def _oracle(q, k, v, bits, group):
    kc, ks, vc, vs = oracle_pack(k, v, bits, group)
    return O.attend_packed(q, kc, ks, vc, vs, k.shape[2], bits, group)


def _attend(q, cache, n, bits, group, **kw):
    return host(kvq.attend(dev(q), *cache, n, bits, group, **kw))


# (B, Hq, Hkv, R, N): rows per KV head 1..8, ragged and block-aligned token
# counts, a head count that is a multiple of 8 (the XCD-aware mapping) and
# some that are not.
SHAPES = [
    (1, 1, 1, 1, 1),        # one token
    (2, 4, 2, 1, 31),       # one partial block
    (1, 8, 2, 1, 33),       # a full block and one token
    (2, 6, 2, 1, 100),      # 3 rows
    (1, 8, 1, 1, 1057),     # 8 rows
    (8, 32, 8, 1, 1000),    # 4 rows, 64 heads
    (2, 4, 1, 2, 700),      # 8 rows from 4 heads x 2 queries
    (3, 10, 2, 1, 513),     # 5 rows, 6 heads
]
FORMATS = [(4, 8), (4, 16), (4, 64), (4, 128), (8, 8), (8, 16), (8, 64), (8, 128)]


def _ids(s):
    return "B{}-Hq{}-Hkv{}-R{}-N{}".format(*s)


@pytest.mark.parametrize("shape", SHAPES, ids=[_ids(s) for s in SHAPES])
@pytest.mark.parametrize("bits,group", FORMATS, ids=[f"{b}b-g{g}" for b, g in FORMATS])
def test_stream_matches_oracle(shape, bits, group):
    B, Hq, Hkv, R, N = shape
    w = Workload("stream", B, Hq, Hkv, R, N, 128, ((bits, group),))
    q, k, v = make_qkv(w, 3)
    announce(f"stream {_ids(shape)} {bits}b g{group}")
    want = _oracle(q, k, v, bits, group)
    cache = _cache(k, v, bits, group)
    general = _attend(q, cache, N, bits, group, variant="valu")
    for splits in (1, 3, 0, 64):
        got = _attend(q, cache, N, bits, group, num_splits=splits, variant="stream")
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))
        assert max_abs(got, general) <= KERNEL_TOL, (splits, max_abs(got, general))


@pytest.mark.parametrize("bits,group", [(4, 8), (8, 16)])
@pytest.mark.parametrize("dist", ["early", "late"])
def test_stream_peaked_scores(bits, group, dist):
    """A few tokens at one end of the cache dominate the softmax (the lazy
    reference has to move once they are reached), and channel scales that
    spread over two decades."""
    w = Workload("stream_peaked", 2, 8, 2, 1, 2000, 128, ((bits, group),), k_channel_scale=True)
    q, k, v = make_qkv(w, 5, dist)
    announce(f"stream peaked {dist} {bits}b g{group}")
    want = _oracle(q, k, v, bits, group)
    cache = _cache(k, v, bits, group)
    for splits in (1, 5, 0):
        got = _attend(q, cache, w.N, bits, group, num_splits=splits, variant="stream")
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


@pytest.mark.parametrize("bits", [4, 8])
def test_stream_group32_equals_matrix_core_path_within_tolerance(bits):
    """Group 32 is served by the matrix-core kernels automatically; the
    streaming kernel forced on it agrees with them and with the oracle."""
    B, Hq, Hkv, R, N = 2, 8, 2, 1, 777
    w = Workload("stream32", B, Hq, Hkv, R, N, 128, ((bits, 32),))
    q, k, v = make_qkv(w, 6)
    announce(f"stream g32 {bits}b")
    want = _oracle(q, k, v, bits, 32)
    cache = _cache(k, v, bits, 32)
    s = _attend(q, cache, N, bits, 32, variant="stream")
    mfma = _attend(q, cache, N, bits, 32, variant="mfma")
    assert max_abs(s, want) <= TOL
    assert max_abs(s, mfma) <= KERNEL_TOL


def test_stream_c4_shape_group8_full():
    """The 8 x 4096-token cache with 32 query heads over 8 KV heads in 4-bit
    group 8, every output against the oracle."""
    base = WORKLOADS["gqa_n4096"]
    w = Workload("gqa_n4096_g8", base.B, base.Hq, base.Hkv, base.R, base.N, base.D, ((4, 8),))
    q, k, v = make_qkv(w, 0)
    announce("stream gqa_n4096 4-bit g8 full")
    want = _oracle(q, k, v, 4, 8)
    cache = _cache(k, v, 4, 8)
    outs = {}
    for splits in (0, 8, 16, 32):
        outs[splits] = _attend(q, cache, w.N, 4, 8, num_splits=splits)
        assert max_abs(outs[splits], want) <= TOL, (splits, max_abs(outs[splits], want))
    for splits in (8, 16, 32):
        assert max_abs(outs[splits], outs[0]) <= KERNEL_TOL


def test_auto_runs_the_streaming_kernel():
    """Where the streaming kernel applies and the matrix-core ones do not,
    the automatic choice gives its output bit for bit."""
    B, Hq, Hkv, R, N = 4, 16, 4, 1, 1500
    for bits, group in ((4, 8), (8, 64)):
        w = Workload("stream_auto", B, Hq, Hkv, R, N, 128, ((bits, group),))
        q, k, v = make_qkv(w, 7)
        announce(f"stream auto {bits}b g{group}")
        cache = _cache(k, v, bits, group)
        qd = dev(q)
        ws = kvq.new_workspace(B, Hq, Hkv, R, N, 128, 0)
        a = kvq.attend(qd, *cache, N, bits, group, workspace=ws)
        b = kvq.attend(qd, *cache, N, bits, group, workspace=ws, variant="stream")
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        assert not torch.any(ws[:256 * B * Hkv])  # split counters back at zero


def test_stream_deterministic_back_to_back():
    """Repeated calls on one workspace give identical bits (fixed reduction
    order, counters reset by every call)."""
    B, Hq, Hkv, R, N = 8, 32, 8, 1, 3000
    w = Workload("stream_det", B, Hq, Hkv, R, N, 128, ((4, 16),))
    q, k, v = make_qkv(w, 8)
    announce("stream determinism")
    cache = _cache(k, v, 4, 16)
    qd = dev(q)
    ws = kvq.new_workspace(B, Hq, Hkv, R, N, 128, 24)
    outs = torch.empty((20,) + tuple(qd.shape), dtype=torch.float32, device="cuda")
    for i in range(20):
        kvq.attend(qd, *cache, N, 4, 16, num_splits=24, workspace=ws, out=outs[i],
                   variant="stream")
    torch.cuda.synchronize()
    same = (outs.view(torch.int32) == outs[0].view(torch.int32)).flatten(1).all(dim=1)
    assert bool(same.all())


@pytest.mark.parametrize("what", ["group2", "group12", "rows9", "d64", "group256"])
def test_stream_variant_rejects_what_it_does_not_take(what):
    B, Hq, Hkv, R, N, D, bits, group = 1, 4, 1, 1, 64, 128, 4, 8
    if what == "group2":
        group = 2
    elif what == "group12":
        group = 12
    elif what == "group256":
        group = 256
    elif what == "rows9":
        Hq = 9
    elif what == "d64":
        D = 64
    q = torch.zeros((B, Hq, R, D), dtype=torch.float32, device="cuda")
    x = torch.zeros((B, Hkv, N, D), dtype=torch.float32, device="cuda")
    kc, ks = kvq.pack_k(x, bits, group)
    vc, vs = kvq.pack_v(x, bits, group)
    with pytest.raises(kvq.KvqError) as e:
        kvq.attend(q, kc, ks, vc, vs, N, bits, group, variant="stream")
    assert e.value.status == -2  # KVQ_ERR_UNSUPPORTED


# Causal chunks on the streaming kernel: (B, Hq, Hkv, R, N), the R queries of
# each head at the last R positions.
CAUSAL_SHAPES = [
    (1, 4, 1, 2, 100),      # 8 rows, the mask inside one block
    (2, 8, 2, 2, 33),       # 8 rows, masked tokens 31 and 32 in two blocks
    (1, 4, 2, 2, 1),        # N < R: query 0 of every head has no legal key
    (2, 2, 2, 4, 1057),     # 4 rows: one head x 4 queries
    (1, 2, 1, 3, 70),       # 6 rows
    (8, 32, 8, 1, 1000),    # R = 1: the unmasked call
]


@pytest.mark.parametrize("shape", CAUSAL_SHAPES, ids=[_ids(s) for s in CAUSAL_SHAPES])
@pytest.mark.parametrize("bits,group", [(4, 8), (8, 16), (4, 64), (8, 128)],
                         ids=["4b-g8", "8b-g16", "4b-g64", "8b-g128"])
def test_stream_causal_matches_oracle(shape, bits, group):
    """Per-row causal limits, rows without a legal key (zeros), masks across two
    blocks and splits past the last token, against the oracle and the general
    kernel; the automatic choice runs the streaming kernel."""
    B, Hq, Hkv, R, N = shape
    w = Workload("stream_causal", B, Hq, Hkv, R, N, 128, ((bits, group),))
    q, k, v = make_qkv(w, 21)
    announce(f"stream causal {_ids(shape)} {bits}b g{group}")
    kc, ks, vc, vs = oracle_pack(k, v, bits, group)
    want = O.attend_packed(q, kc, ks, vc, vs, N, bits, group, causal=True)
    empty = O.causal_mask(N, R).sum(axis=1) == 0       # queries with no legal key
    cache = _cache(k, v, bits, group)
    for splits in (1, 3, 0, 64):
        got = _attend(q, cache, N, bits, group, num_splits=splits, variant="stream", causal=True)
        assert np.isfinite(got).all(), splits
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))
        assert (got[:, :, empty] == 0).all(), splits
        gen = _attend(q, cache, N, bits, group, num_splits=splits, variant="valu", causal=True)
        assert max_abs(got, gen) <= KERNEL_TOL, (splits, max_abs(got, gen))
    auto = _attend(q, cache, N, bits, group, causal=True)
    stream = _attend(q, cache, N, bits, group, variant="stream", causal=True)
    assert np.array_equal(auto, stream)
