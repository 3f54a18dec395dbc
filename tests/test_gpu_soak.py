"""Bounded soak of the fused attend on the 8 x 4096-token cache (the timed
decode configuration), and of the 32-row kernel on a GQA 64/8 cache with 4
queries per head.  Each split count runs 2000 (600) back-to-back calls
through one workspace, alternating two copies of the packed cache.  Every
output must be bit-identical to the first call's.  The check runs in batches
of 100 calls written into NaN-filled buffers, so an output left unwritten
also fails, and the first mismatching call is named.

This exercises the split combine's counters on every call: each call resets
them for the next, with no host-side clearing in between."""
import pytest

from workloads import WORKLOADS, Workload, make_qkv

from gpu_helpers import announce, dev

pytestmark = pytest.mark.gpu

kvq = pytest.importorskip("quantized_kv_cache_attend_amd")
torch = pytest.importorskip("torch")

CALLS = 2000
BATCH = 100


@pytest.mark.parametrize("splits", [4, 16, 64])
def test_soak_gqa_n4096(splits):
    w = WORKLOADS["gqa_n4096"]
    bits, group = w.formats[0]
    q, k, v = make_qkv(w, 0)
    qd = dev(q)
    kc, ks = kvq.pack_k(dev(k), bits, group)
    vc, vs = kvq.pack_v(dev(v), bits, group)
    caches = [(kc, ks, vc, vs), tuple(t.clone() for t in (kc, ks, vc, vs))]
    ws = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D, splits, device="cuda")
    announce(f"soak gqa_n4096 splits={splits} calls={CALLS}")
    first = kvq.attend(qd, *caches[0], w.N, bits, group, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(first).all())
    first_bits = first.view(torch.int32)
    outs = torch.empty((BATCH,) + tuple(qd.shape), dtype=torch.float32, device="cuda")
    done = 0
    while done < CALLS:
        n = min(BATCH, CALLS - done)
        outs.fill_(float("nan"))
        for i in range(n):
            kvq.attend(qd, *caches[(done + i) % 2], w.N, bits, group, num_splits=splits,
                       workspace=ws, out=outs[i])
        torch.cuda.synchronize()
        same = (outs[:n].view(torch.int32) == first_bits).flatten(1).all(dim=1)
        if not bool(same.all()):
            bad = int(torch.nonzero(~same)[0, 0])
            pytest.fail(f"call {done + bad + 1} of {CALLS} (splits={splits}) differs from the first")
        done += n


# GQA 64/8 with 4 queries per head (32 rows per KV head, the 32-row
# matrix-core kernel) on 4 x 8192 tokens.  16 splits put 4 splits in each
# workgroup, one per wave (the two-level combine); 4 splits one per
# workgroup; 64 splits take two rounds of workgroups.  The waves' issue
# priorities change with the blocks each has left, so arrival order varies
# from call to call while the merge order must not.
ROWS32 = Workload("soak_rows32", 4, 64, 8, 4, 8192, 128, ((4, 32),))
CALLS32 = 600


@pytest.mark.parametrize("bits,splits", [(4, 16), (4, 4), (8, 16), (4, 64)])
def test_soak_rows32(bits, splits):
    w = ROWS32
    q, k, v = make_qkv(w, 1)
    qd = dev(q)
    kc, ks = kvq.pack_k(dev(k), bits, 32)
    vc, vs = kvq.pack_v(dev(v), bits, 32)
    caches = [(kc, ks, vc, vs), tuple(t.clone() for t in (kc, ks, vc, vs))]
    ws = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D, splits, device="cuda")
    announce(f"soak rows32 bits={bits} splits={splits} calls={CALLS32}")
    first = kvq.attend(qd, *caches[0], w.N, bits, 32, num_splits=splits, workspace=ws,
                       variant="mfma")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(first).all())
    first_bits = first.view(torch.int32)
    outs = torch.empty((BATCH,) + tuple(qd.shape), dtype=torch.float32, device="cuda")
    done = 0
    while done < CALLS32:
        n = min(BATCH, CALLS32 - done)
        outs.fill_(float("nan"))
        for i in range(n):
            kvq.attend(qd, *caches[(done + i) % 2], w.N, bits, 32, num_splits=splits,
                       workspace=ws, out=outs[i], variant="mfma")
        torch.cuda.synchronize()
        same = (outs[:n].view(torch.int32) == first_bits).flatten(1).all(dim=1)
        if not bool(same.all()):
            bad = int(torch.nonzero(~same)[0, 0])
            pytest.fail(f"call {done + bad + 1} of {CALLS32} (bits={bits}, splits={splits}) "
                        "differs from the first")
        done += n
