"""kvq_attend_noalloc (the library's own scratch in place of a caller
workspace) called through the C ABI, against kvq_attend on the same inputs:
a sequence of calls on one GPU whose (batch, KV head) count shrinks and grows
again, every result equal to kvq_attend's and within 1e-4 of the oracle."""
import ctypes

import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import WORKLOADS, Workload, make_qkv

from gpu_helpers import announce, dev, host, max_abs, oracle_pack

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")
torch = pytest.importorskip("torch")

TOL = 1e-4


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _noalloc(qd, cache, w, bits, group, splits, out):
    return kvq.lib.kvq_attend_noalloc(_p(qd), *[_p(t) for t in cache], w.B, w.Hq, w.Hkv, w.R,
                                      w.N, w.D, bits, group, 0.0, splits, _p(out), _stream())


# (workload, bits, group, splits): the 8 x 4096-token cache, then smaller
# calls (fewer (batch, KV head) pairs: their partials overwrite counters of the
# larger one), a 32-row GQA shape, the general kernel, the streaming kernel
# (group 8, automatic splits), and the large one again.
SEQUENCE = [
    (WORKLOADS["gqa_n4096"], 4, 32, 0),
    (Workload("small", 1, 4, 1, 1, 1000, 128, ((4, 32),)), 4, 32, 3),
    (Workload("rows32", 2, 16, 2, 4, 3000, 128, ((4, 32),)), 4, 32, 0),
    (Workload("valu", 1, 4, 2, 2, 700, 32, ((4, 8),)), 4, 8, 5),
    (Workload("r4_8bit", 4, 8, 4, 1, 2000, 128, ((8, 32),)), 8, 32, 4),
    (Workload("stream", 2, 8, 2, 1, 1500, 128, ((4, 8),)), 4, 8, 0),
    (WORKLOADS["gqa_n4096"], 4, 32, 8),
]


def test_noalloc_matches_kvq_attend():
    for i, (w, bits, group, splits) in enumerate(SEQUENCE):
        q, k, v = make_qkv(w, 20 + i)
        announce(f"attend_noalloc step {i}: {w.name} {bits}b g{group} splits={splits}")
        qd = dev(q)
        cache = kvq.pack_k(dev(k), bits, group) + kvq.pack_v(dev(v), bits, group)
        want = host(kvq.attend(qd, *cache, w.N, bits, group, num_splits=splits))
        out = torch.full_like(qd, float("nan"))
        st = _noalloc(qd, cache, w, bits, group, splits, out)
        assert st == kvq.KVQ_OK, kvq.lib.kvq_last_error()
        got = host(out)
        assert np.array_equal(got, want), (i, max_abs(got, want))
        okc, oks, ovc, ovs = oracle_pack(k, v, bits, group)
        assert max_abs(got, O.attend_packed(q, okc, oks, ovc, ovs, w.N, bits, group)) <= TOL
    # the binding's wrapper is the same call
    w, bits, group, splits = SEQUENCE[1]
    q, k, v = make_qkv(w, 21)
    cache = kvq.pack_k(dev(k), bits, group) + kvq.pack_v(dev(v), bits, group)
    got = host(kvq.attend_noalloc(dev(q), *cache, w.N, bits, group, num_splits=splits))
    want = host(kvq.attend(dev(q), *cache, w.N, bits, group, num_splits=splits))
    assert np.array_equal(got, want)


def test_noalloc_rejects_more_than_its_scratch():
    """The 32768-token workload with its 16 splits needs 34 MB of partials,
    more than the 16 MiB scratch: KVQ_ERR_WORKSPACE before anything runs
    (the array pointers are never touched)."""
    w = WORKLOADS["gqa_n32768"]
    fake = [ctypes.c_void_p(i << 40) for i in range(1, 6)]
    out = ctypes.c_void_p(7 << 40)
    st = kvq.lib.kvq_attend_noalloc(*fake, w.B, w.Hq, w.Hkv, w.R, w.N, w.D, 4, 32, 0.0, 16, out,
                                    _stream())
    assert st == kvq.KVQ_ERR_WORKSPACE
    assert b"scratch" in kvq.lib.kvq_last_error()
