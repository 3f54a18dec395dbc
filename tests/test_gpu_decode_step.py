"""One-call decode step (kvq_append_attend) against the two calls it stands
for, kvq_append of one token and then kvq_attend_cache over the N + 1
tokens: the cache arrays, k_tail and the output must match bit for bit after
every step, across group boundaries and from an empty cache, both where one
launch does both (the 4-row matrix-core kernel, with the append in extra
workgroups) and where the call falls back to two launches.  The last step's
output is also checked against the float64 oracle over the packed prefix
([RL] "prefill and decode": a decode step reads the cached K/V and appends
its new position)."""
import pytest

from oracle import kvq_oracle as O
from workloads import Workload, make_qkv

from gpu_helpers import announce, dev, host, max_abs

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")
torch = pytest.importorskip("torch")

TOL = 1e-4

# (B, Hq, Hkv, R, bits, group, num_splits, first N, steps)
CASES = [
    (8, 32, 8, 1, 4, 32, 0, 90, 40),    # 64 heads (a multiple of 8), automatic splits
    (2, 6, 3, 1, 4, 32, 3, 0, 40),      # 6 heads, 3 splits, from an empty cache
    (1, 4, 1, 1, 8, 32, 1, 29, 6),      # 8-bit, one split (no combine), across token 32
    (2, 4, 2, 1, 8, 32, 0, 60, 10),     # 8-bit, automatic splits
    (2, 8, 2, 2, 4, 32, 0, 60, 10),     # 8 rows per KV head: the 32-row kernel, two launches
    (2, 8, 2, 1, 4, 8, 2, 60, 10),      # group 8: append, then the streaming kernel (two launches)
    (1, 8, 1, 1, 8, 16, 0, 5, 40),      # 8-bit group 16, 8 rows: the streaming kernel, auto splits
]


def _ids(c):
    return "B{}-Hq{}-Hkv{}-R{}-{}b-g{}-s{}-N{}+{}".format(*c)


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_decode_step_equals_append_then_attend(case):
    B, Hq, Hkv, R, bits, group, splits, n0, steps = case
    D = 128
    cap = n0 + steps + 7
    w = Workload("dstep", B, Hq, Hkv, R, n0 + steps, D, ((bits, group),))
    q, k, v = make_qkv(w, 13)
    announce(f"decode step {_ids(case)}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    caches = [kvq.new_cache(B, Hkv, cap, D, bits, group) for _ in range(2)]
    if n0:
        for c in caches:
            kvq.append(kd[:, :, :n0].contiguous(), vd[:, :, :n0].contiguous(), 0, c, cap, bits,
                       group)
    ws = [kvq.new_workspace(B, Hq, Hkv, R, cap, D, splits) for _ in range(2)]
    for i in range(steps):
        n = n0 + i
        kt = kd[:, :, n:n + 1].contiguous()
        vt = vd[:, :, n:n + 1].contiguous()
        kvq.append(kt, vt, n, caches[0], cap, bits, group)
        ref = kvq.attend(qd, *caches[0][:4], n + 1, bits, group, num_splits=splits,
                         workspace=ws[0], capacity=cap)
        got = kvq.append_attend(qd, kt, vt, n, caches[1], cap, bits, group, num_splits=splits,
                                workspace=ws[1])
        torch.cuda.synchronize()
        names = ("k_codes", "k_scales", "v_codes", "v_scales", "k_tail")
        for name, a, b in zip(names, caches[0], caches[1]):
            assert torch.equal(a, b), (i, n, name)
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), (i, n)
    # the last step against the oracle over the packed prefix
    n1 = n0 + steps
    kc, ks = O.pack_k(k[:, :, :n1], bits, group)
    vc, vs = O.pack_v(v[:, :, :n1], bits, group)
    want = O.attend_packed(q, kc, ks, vc, vs, n1, bits, group)
    assert max_abs(host(got), want) <= TOL


def test_decode_step_back_to_back_one_workspace():
    """Many fused steps back to back on one workspace, without host syncs in
    between (the append flag and split counters must be reset by every call),
    bit-identical to the two-call path run the same way."""
    B, Hq, Hkv, R, bits, group = 8, 32, 8, 1, 4, 32
    D, n0, steps = 128, 200, 64
    cap = n0 + steps
    w = Workload("dstep2", B, Hq, Hkv, R, cap, D, ((bits, group),))
    q, k, v = make_qkv(w, 14)
    announce("decode step back to back, 64 steps")
    qd, kd, vd = dev(q), dev(k), dev(v)
    caches = [kvq.new_cache(B, Hkv, cap, D, bits, group) for _ in range(2)]
    for c in caches:
        kvq.append(kd[:, :, :n0].contiguous(), vd[:, :, :n0].contiguous(), 0, c, cap, bits, group)
    ws = [kvq.new_workspace(B, Hq, Hkv, R, cap, D, 0) for _ in range(2)]
    outs = torch.empty((2, steps) + tuple(qd.shape), dtype=torch.float32, device="cuda")
    rows = [(kd[:, :, n:n + 1].contiguous(), vd[:, :, n:n + 1].contiguous())
            for n in range(n0, cap)]
    for i, (kt, vt) in enumerate(rows):
        kvq.append(kt, vt, n0 + i, caches[0], cap, bits, group)
        kvq.attend(qd, *caches[0][:4], n0 + i + 1, bits, group, workspace=ws[0], capacity=cap,
                   out=outs[0, i])
    for i, (kt, vt) in enumerate(rows):
        kvq.append_attend(qd, kt, vt, n0 + i, caches[1], cap, bits, group, workspace=ws[1],
                          out=outs[1, i])
    torch.cuda.synchronize()
    for a, b in zip(caches[0], caches[1]):
        assert torch.equal(a, b)
    same = (outs[0].view(torch.int32) == outs[1].view(torch.int32)).flatten(1).all(dim=1)
    assert bool(same.all()), int(torch.nonzero(~same)[0, 0])
    assert torch.all(ws[1][:256 * B * Hkv] == 0)  # counters and append flags back at zero


def test_decode_step_rejects_bad_arguments():
    B, Hq, Hkv, R, D = 1, 4, 1, 1, 128
    q = torch.zeros((B, Hq, R, D), dtype=torch.float32, device="cuda")
    kt = torch.zeros((B, Hkv, 1, D), dtype=torch.float32, device="cuda")
    cache = kvq.new_cache(B, Hkv, 32, D, 4, 32)
    with pytest.raises(kvq.KvqError):   # N + 1 > capacity
        kvq.append_attend(q, kt, kt, 32, cache, 32, 4, 32)
    with pytest.raises(ValueError):     # the new rows must be [B, Hkv, 1, D]
        kvq.append_attend(q, kt.expand(B, Hkv, 2, D).contiguous(), kt, 3, cache, 32, 4, 32)
