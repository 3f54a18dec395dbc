"""GPU tests of the boundary itself: the float32-cache attend at every
compiled head dimension, the C-ABI entry point kvq_attend called directly,
guard bytes around every kernel family's output and workspace, argument
checks of the binding, and workspaces reused across call shapes."""
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


def _unaligned(a):
    """A contiguous device copy of `a` starting 4 bytes past a 16-byte boundary."""
    flat = torch.zeros(a.size + 1, dtype=torch.float32, device="cuda")
    view = flat[1:].view(a.shape)
    view.copy_(torch.from_numpy(np.ascontiguousarray(a)))
    assert view.data_ptr() % 16 == 4
    return view


# --- kvq_attend_f32 (the float32-cache path and the attend half of decode-all) -------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 37, 1021, 4097])
@pytest.mark.parametrize("hq,hkv,r", [(1, 1, 4), (8, 2, 2), (32, 8, 1)])
def test_attend_f32_head_dims(d, n, hq, hkv, r):
    """[BKD] "Compare equivalent representations first": attention over the
    float32 cache, at the head dims the decode-all baseline is timed on, for
    ragged token counts, GQA shapes and split counts, with the float32 rows
    16-byte aligned (whole-row loads) and 4 bytes off (element loads)."""
    w = Workload("f32", 2, hq, hkv, r, n, d, ((4, 32),))
    q, k, v = make_qkv(w, 11)
    announce(f"attend_f32 d={d} n={n} hq={hq} hkv={hkv} r={r}")
    want = O.attend_dense(q, k, v)
    qd, kd, vd = dev(q), dev(k), dev(v)
    for splits in (1, 3, 0):
        got = host(kvq.attend_f32(qd, kd, vd, num_splits=splits))
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))
    got = host(kvq.attend_f32(qd, _unaligned(k), _unaligned(v), num_splits=3))
    assert max_abs(got, want) <= TOL


def test_decode_all_gqa_n4096():
    """Decode-all on the 8 x 4096-token cache (the shape bench.py times):
    kvq_dequant_k/_v write float32 K and V, kvq_attend_f32 attends them; the
    result is the oracle's attention over the same quantized cache."""
    w = WORKLOADS["gqa_n4096"]
    q, k, v = make_qkv(w, 0)
    announce("decode-all gqa_n4096")
    kc, ks = kvq.pack_k(dev(k), 4, 32)
    vc, vs = kvq.pack_v(dev(v), 4, 32)
    kf = kvq.dequant_k(kc, ks, w.N, w.D, 4, 32)
    vf = kvq.dequant_v(vc, vs, w.N, w.D, 4, 32)
    okc, oks, ovc, ovs = oracle_pack(k, v, 4, 32)
    want = O.attend_packed(q, okc, oks, ovc, ovs, w.N, 4, 32)
    for splits in (0, 8):
        got = host(kvq.attend_f32(dev(q), kf, vf, num_splits=splits))
        assert max_abs(got, want) <= TOL, (splits, max_abs(got, want))


# --- the C-ABI entry point kvq_attend, called through ctypes -----------------------------

def test_kvq_attend_direct_c_abi_gqa_n4096():
    """kvq_attend (the header's plain entry point, automatic kernel choice) on
    the full 8 x 4096-token cache, called with raw device pointers and the
    current stream: the result is the oracle's within 1e-4, and an explicit
    split count gives the same result within 2e-5."""
    w = WORKLOADS["gqa_n4096"]
    q, k, v = make_qkv(w, 1)
    announce("kvq_attend direct gqa_n4096")
    kc, ks = kvq.pack_k(dev(k), 4, 32)
    vc, vs = kvq.pack_v(dev(v), 4, 32)
    qd = dev(q)
    outs = []
    for splits in (0, 4):
        nbytes = kvq.lib.kvq_attend_workspace_bytes(w.B, w.Hq, w.Hkv, w.R, w.N, w.D, splits)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(qd)
        st = kvq.lib.kvq_attend(
            ctypes.c_void_p(qd.data_ptr()), ctypes.c_void_p(kc.data_ptr()),
            ctypes.c_void_p(ks.data_ptr()), ctypes.c_void_p(vc.data_ptr()),
            ctypes.c_void_p(vs.data_ptr()), w.B, w.Hq, w.Hkv, w.R, w.N, w.D, 4, 32, 0.0, splits,
            ctypes.c_void_p(ws.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == kvq.KVQ_OK, kvq.lib.kvq_last_error()
        torch.cuda.synchronize()
        outs.append(host(out))
        # every completed call leaves the arrival counters zero
        assert not host(ws)[:256 * w.B * w.Hkv].any()
    okc, oks, ovc, ovs = oracle_pack(k, v, 4, 32)
    want = O.attend_packed(q, okc, oks, ovc, ovs, w.N, 4, 32)
    assert max_abs(outs[0], want) <= TOL
    assert max_abs(outs[1], outs[0]) <= 2e-5


# --- guard bytes around the output and the workspace ------------------------------------

SENTINEL = np.float32(-1234.5)
GUARD = 1024  # floats (4 KB) on each side of out, bytes after the workspace


def _guarded_out(shape):
    n = int(np.prod(shape))
    big = torch.full((n + 2 * GUARD,), float(SENTINEL), dtype=torch.float32, device="cuda")
    return big, big[GUARD:GUARD + n].view(shape)


def _guarded_ws(nbytes):
    big = torch.zeros(nbytes + 4096, dtype=torch.uint8, device="cuda")
    return big, big[:nbytes]


def _check_guards(big_out, n, big_ws, nbytes):
    h = host(big_out)
    assert np.all(h[:GUARD] == SENTINEL) and np.all(h[GUARD + n:] == SENTINEL), "out guard written"
    assert not host(big_ws)[nbytes:].any(), "workspace guard written"


FAMILIES = [
    # name, workload (B, Hq, Hkv, R, N, D), bits, group, variant, causal, splits
    ("valu", (2, 8, 2, 2, 1000, 32), 4, 8, "valu", False, 3),
    ("valu-causal", (2, 8, 2, 3, 1000, 64), 8, 32, "valu", True, 5),
    ("mfma-r4", (2, 8, 2, 1, 1000, 128), 4, 32, "mfma", False, 3),
    ("mfma-r4-8bit", (2, 8, 2, 1, 1000, 128), 8, 32, "mfma", False, 2),
    ("mfma-r8-8bit", (2, 8, 2, 2, 1000, 128), 8, 32, "mfma", False, 2),
    ("mfma-r32", (2, 16, 2, 4, 1000, 128), 4, 32, "mfma", False, 3),
    ("mfma-r32-causal", (2, 16, 2, 4, 1000, 128), 4, 32, "mfma", True, 4),
    ("mfma-r16-8bit", (2, 8, 2, 4, 1000, 128), 8, 32, "mfma", False, 1),
]


@pytest.mark.parametrize("name,shape,bits,group,variant,causal,splits", FAMILIES)
def test_guard_bytes_packed(name, shape, bits, group, variant, causal, splits):
    """Each kernel family writes exactly its output rows and stays inside the
    workspace size it asked for: 4 KB of sentinel floats before and after
    `out`, and zeros past the workspace, are unchanged after the call."""
    B, Hq, Hkv, R, N, D = shape
    w = Workload(name, B, Hq, Hkv, R, N, D, ((bits, group),))
    q, k, v = make_qkv(w, 12)
    announce(f"guard bytes {name}")
    kc, ks = kvq.pack_k(dev(k), bits, group)
    vc, vs = kvq.pack_v(dev(v), bits, group)
    big_out, out = _guarded_out(q.shape)
    nbytes = kvq.workspace_bytes(B, Hq, Hkv, R, N, D, splits)
    big_ws, ws = _guarded_ws(nbytes)
    kvq.attend(dev(q), kc, ks, vc, vs, N, bits, group, num_splits=splits, workspace=ws, out=out,
               variant=variant, capacity=N if causal else None, causal=causal)
    torch.cuda.synchronize()
    _check_guards(big_out, q.size, big_ws, nbytes)
    okc, oks, ovc, ovs = oracle_pack(k, v, bits, group)
    want = O.attend_packed(q, okc, oks, ovc, ovs, N, bits, group, causal=causal)
    assert max_abs(host(out), want) <= TOL


def test_guard_bytes_f32_and_window():
    """The same guards around the float32-cache attend and both forms of the
    mixed cache (fused into the matrix-core launch with 16-byte-aligned window
    rows, and the general kernel when the rows are 4 bytes off)."""
    B, Hq, Hkv, R, N, D, W = 2, 8, 2, 2, 900, 128, 40
    w = Workload("gw", B, Hq, Hkv, R, N + W, D, ((4, 32),))
    q, k, v = make_qkv(w, 13)
    announce("guard bytes f32 / window")
    big_out, out = _guarded_out(q.shape)
    nbytes = kvq.workspace_bytes(B, Hq, Hkv, R, N + W, D, 3)
    big_ws, ws = _guarded_ws(nbytes)
    kvq.attend_f32(dev(q), dev(k), dev(v), num_splits=3, workspace=ws, out=out)
    torch.cuda.synchronize()
    _check_guards(big_out, q.size, big_ws, nbytes)
    assert max_abs(host(out), O.attend_dense(q, k, v)) <= TOL

    kc, ks = kvq.pack_k(dev(k[:, :, :N].copy()), 4, 32)
    vc, vs = kvq.pack_v(dev(v[:, :, :N].copy()), 4, 32)
    want = O.attend_window(q, k, v, W, 4, 32)
    slots = 3 + (W + 31) // 32
    for kw_, vw_ in ((dev(k[:, :, N:].copy()), dev(v[:, :, N:].copy())),
                     (_unaligned(k[:, :, N:].copy()), _unaligned(v[:, :, N:].copy()))):
        big_out, out = _guarded_out(q.shape)
        nbytes = kvq.workspace_bytes(B, Hq, Hkv, R, N + W, D, slots)
        big_ws, ws = _guarded_ws(nbytes)
        kvq.attend_window(dev(q), kc, ks, vc, vs, kw_, vw_, N, 4, 32, num_splits=3, workspace=ws,
                          out=out)
        torch.cuda.synchronize()
        _check_guards(big_out, q.size, big_ws, nbytes)
        assert max_abs(host(out), want) <= TOL


# --- argument checks of the binding (before any launch) -----------------------------------

def test_binding_rejects_bad_out_and_workspace():
    w = WORKLOADS["single_n128"]
    q, k, v = make_qkv(w, 0)
    kc, ks = kvq.pack_k(dev(k), 4, 32)
    vc, vs = kvq.pack_v(dev(v), 4, 32)
    qd = dev(q)
    ws = kvq.new_workspace(w.B, w.Hq, w.Hkv, w.R, w.N, w.D)
    bad_outs = [torch.empty(q.shape, dtype=torch.float16, device="cuda"),
                torch.empty((q.size - 1,), dtype=torch.float32, device="cuda"),
                torch.empty(q.shape[:2] + (q.shape[3], q.shape[2]), dtype=torch.float32,
                            device="cuda").transpose(2, 3),          # not contiguous
                torch.empty(q.shape, dtype=torch.float32)]
    for out in bad_outs:
        with pytest.raises((TypeError, ValueError)):
            kvq.attend(qd, kc, ks, vc, vs, w.N, 4, 32, workspace=ws, out=out)
        with pytest.raises((TypeError, ValueError)):
            kvq.attend_f32(qd, dev(k), dev(v), workspace=ws, out=out)
    with pytest.raises((TypeError, ValueError)):
        kvq.attend(qd, kc, ks, vc, vs, w.N, 4, 32, workspace=torch.zeros(4096, dtype=torch.uint8))
    with pytest.raises(ValueError):
        kvq.attend_f32(qd, dev(k), dev(v[:, :, :64].copy()))
    with pytest.raises(ValueError):
        kvq.attend_f32(qd, dev(k[:, :, :, :16].copy()), dev(v[:, :, :, :16].copy()))
    with pytest.raises(kvq.KvqError) as e:   # workspace too small for the split count
        kvq.attend(qd, kc, ks, vc, vs, w.N, 4, 32, num_splits=4,
                   workspace=torch.zeros(256, dtype=torch.uint8, device="cuda"))
    assert e.value.status == kvq.KVQ_ERR_WORKSPACE


# --- one workspace across call shapes ---------------------------------------------------

def test_workspace_reused_for_more_heads():
    """A workspace that served a call with one (batch, KV head) pair may hold
    that call's partial sums where a call with eight pairs keeps its arrival
    counters (here: every byte past the first counter set non-zero, as such
    partials can leave it).  Through the binding the new counter range is
    zero-filled first and the larger call is right, also after a smaller call
    in between.  Called through the C ABI on the same dirty workspace, every
    head whose counter is not zero gets NaN outputs (the stale counter is
    detected, not merged early or never), and the head with a zero counter is
    right."""
    small = Workload("ws1", 1, 4, 1, 1, 2048, 128, ((4, 32),))
    big = Workload("ws8", 2, 16, 4, 1, 2048, 128, ((4, 32),))
    splits = 4
    nbytes = max(kvq.workspace_bytes(1, 4, 1, 1, 2048, 128, splits),
                 kvq.workspace_bytes(2, 16, 4, 1, 2048, 128, splits))
    announce("workspace reuse")
    qs, ks_, vs_ = make_qkv(small, 14)
    qb, kb, vb = make_qkv(big, 15)
    cs = kvq.pack_k(dev(ks_), 4, 32) + kvq.pack_v(dev(vs_), 4, 32)
    cb = kvq.pack_k(dev(kb), 4, 32) + kvq.pack_v(dev(vb), 4, 32)
    okc, oks, ovc, ovs = oracle_pack(kb, vb, 4, 32)
    want = O.attend_packed(qb, okc, oks, ovc, ovs, big.N, 4, 32)

    # binding: the larger call's counters are cleared before it runs
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    kvq.attend(dev(qs), *cs, small.N, num_splits=splits, workspace=ws)
    ws[256:].fill_(0x3F)
    got = host(kvq.attend(dev(qb), *cb, big.N, num_splits=splits, workspace=ws))
    assert max_abs(got, want) <= TOL
    # large, small (dirtying the large call's counters of heads 1..7), large again
    kvq.attend(dev(qs), *cs, small.N, num_splits=splits, workspace=ws)
    ws[256:].fill_(0x3F)
    got2 = host(kvq.attend(dev(qb), *cb, big.N, num_splits=splits, workspace=ws))
    assert np.array_equal(got2, got)

    # C ABI: the same dirty workspace without the clearing
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ws[256:].fill_(0x3F)
    torch.cuda.synchronize()
    counters = host(ws)[:256 * 8].view(np.uint32)[::64].copy()
    assert counters[0] == 0 and np.all(counters[1:] >= splits)
    qd = dev(qb)
    out = torch.empty_like(qd)
    st = kvq.lib.kvq_attend_variant(
        ctypes.c_void_p(qd.data_ptr()), *[ctypes.c_void_p(t.data_ptr()) for t in cb], 2, 16, 4, 1,
        big.N, 128, 4, 32, 0.0, splits, ctypes.c_void_p(ws.data_ptr()), nbytes,
        ctypes.c_void_p(out.data_ptr()), kvq.VARIANTS["mfma"],
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == kvq.KVQ_OK
    got = host(out).reshape(2 * 4, 4, 128)       # [(b, kv head), rows, D]
    ref = want.reshape(2 * 4, 4, 128)
    assert max_abs(got[0], ref[0]) <= TOL
    for h in range(1, 8):
        assert np.all(np.isnan(got[h])), h
