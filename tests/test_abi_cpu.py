"""Host-side tests of the C ABI that need no GPU: the library loads, exports
every function include/kvq.h declares, sizes the packed arrays like the
oracle does, and rejects bad arguments before any work reaches a device."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import kvq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

kvq = pytest.importorskip("quantized_kv_cache_attend_amd",
                          reason="libkvq.so not built (python -m quantized_kv_cache_attend_amd.build)")
lib = kvq.lib

FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: every call below fails validation first
FAKE2 = ctypes.c_void_p(0x20000000)


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name
        assert name in kvq._SIGNATURES, f"binding lacks {name}"


def test_abi_version_and_strings():
    assert lib.kvq_abi_version() == 10
    for st in (0, -1, -2, -3, -4, 7):
        assert lib.kvq_status_string(st)


@pytest.mark.parametrize("N,D", [(128, 32), (512, 32), (35, 13), (1, 1), (4096, 128)])
@pytest.mark.parametrize("bits,group", [(4, 8), (4, 32), (8, 8), (8, 32), (4, 2)])
def test_sizes_match_oracle_arrays(N, D, bits, group):
    x = np.zeros((2, 3, N, D), np.float32)
    kc, ks = O.store_k(*O.pack_k(x, bits, group), N, D, bits, group)
    vc, vs = O.store_v(*O.pack_v(x, bits, group), N, D, bits, group)
    assert lib.kvq_k_code_bytes(2, 3, N, D, bits, group) == kc.nbytes
    assert lib.kvq_k_scale_count(2, 3, N, D, bits, group) == ks.size
    assert lib.kvq_v_code_bytes(2, 3, N, D, bits, group) == vc.nbytes
    assert lib.kvq_v_scale_count(2, 3, N, D, bits, group) == vs.size
    shapes = kvq.packed_shapes(2, 3, N, D, bits, group)
    assert shapes == (kc.shape, ks.shape, vc.shape, vs.shape)


def test_sizes_reject_bad_format():
    assert lib.kvq_k_code_bytes(1, 1, 128, 32, 3, 32) == 0
    assert lib.kvq_k_code_bytes(1, 1, 128, 32, 4, 7) == 0
    assert lib.kvq_v_scale_count(1, 1, 0, 32, 4, 32) == 0


def test_auto_splits_and_workspace():
    # about 512 workgroups, never splits shorter than 512 tokens
    assert lib.kvq_attend_auto_splits(8, 8, 4096) == 8
    assert lib.kvq_attend_auto_splits(1, 1, 128) == 4       # one 32-token tile per split
    assert lib.kvq_attend_auto_splits(1, 1, 1024) == 32
    assert lib.kvq_attend_auto_splits(1, 1, 31) == 1
    assert lib.kvq_attend_auto_splits(1, 1, 1 << 20) == 512
    assert lib.kvq_attend_auto_splits(16, 8, 32768) == 4
    w1 = lib.kvq_attend_workspace_bytes(8, 32, 8, 1, 4096, 128, 8)
    rows = 8 * 32 * 1
    assert w1 >= 8 * rows * (128 + 2) * 4 + 8 * 8 * 4
    assert w1 % 256 == 0
    assert lib.kvq_attend_workspace_bytes(8, 32, 8, 1, 4096, 128, 0) == w1


def _attend(**kw):
    a = dict(q=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, B=1, Hq=4, Hkv=2, R=1, N=64, D=32,
             bits=4, group=32, sm=0.0, splits=1, ws=None, wsb=0, out=FAKE2, variant=0)
    a.update(kw)
    return lib.kvq_attend_variant(a["q"], a["kc"], a["ks"], a["vc"], a["vs"], a["B"], a["Hq"],
                                  a["Hkv"], a["R"], a["N"], a["D"], a["bits"], a["group"],
                                  a["sm"], a["splits"], a["ws"], a["wsb"], a["out"], a["variant"],
                                  None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), kvq.KVQ_ERR_INVALID),
    (dict(N=0), kvq.KVQ_ERR_INVALID),
    (dict(Hq=3), kvq.KVQ_ERR_INVALID),
    (dict(bits=5), kvq.KVQ_ERR_INVALID),
    (dict(group=7), kvq.KVQ_ERR_INVALID),
    (dict(splits=-1), kvq.KVQ_ERR_INVALID),
    (dict(sm=float("nan")), kvq.KVQ_ERR_INVALID),
    (dict(out=FAKE), kvq.KVQ_ERR_INVALID),                    # aliases q
    (dict(q=ctypes.c_void_p(0x10002)), kvq.KVQ_ERR_INVALID),  # misaligned float pointer
    (dict(D=48), kvq.KVQ_ERR_UNSUPPORTED),
    (dict(Hq=128, Hkv=1), kvq.KVQ_ERR_UNSUPPORTED),          # 128 rows per KV head
    (dict(splits=4), kvq.KVQ_ERR_WORKSPACE),                 # no workspace
    (dict(splits=4, ws=ctypes.c_void_p(0x40000000), wsb=64), kvq.KVQ_ERR_WORKSPACE),
    (dict(variant=9), kvq.KVQ_ERR_INVALID),
    (dict(variant=2, bits=8), kvq.KVQ_ERR_UNSUPPORTED),      # matrix-core kernels: D = 128 only
    (dict(variant=2, D=128, group=8, out=ctypes.c_void_p(1 << 44)),
     kvq.KVQ_ERR_UNSUPPORTED),                              # and group 32 only
    (dict(variant=2, D=128, bits=8, N=(1 << 24) - 31, out=ctypes.c_void_p(1 << 44)),
     kvq.KVQ_ERR_UNSUPPORTED),                              # 8-bit: 4 KB blocks, half the tokens
    (dict(variant=2, D=128, N=(1 << 25) - 31, out=ctypes.c_void_p(1 << 44)),
     kvq.KVQ_ERR_UNSUPPORTED),                              # past its 32-bit buffer offsets
])
def test_attend_rejects_before_launch(kw, status):
    assert _attend(**kw) == status
    assert lib.kvq_last_error()


def test_codec_rejects_before_launch():
    for fn in (lib.kvq_pack_k, lib.kvq_pack_v):
        assert fn(None, 1, 1, 8, 8, 4, 8, FAKE, FAKE2, None) == kvq.KVQ_ERR_INVALID
        assert fn(FAKE, 1, 1, 8, 8, 4, 3, FAKE, FAKE2, None) == kvq.KVQ_ERR_INVALID
        assert fn(FAKE, 1, 0, 8, 8, 4, 8, FAKE, FAKE2, None) == kvq.KVQ_ERR_INVALID
    for fn in (lib.kvq_dequant_k, lib.kvq_dequant_v):
        assert fn(FAKE, None, 1, 1, 8, 8, 4, 8, FAKE2, None) == kvq.KVQ_ERR_INVALID
        assert fn(FAKE, FAKE2, 1, 1, 8, 8, 6, 8, FAKE2, None) == kvq.KVQ_ERR_INVALID
        # 32-bit element index per head
        assert fn(FAKE, FAKE2, 1, 1, 1 << 25, 128, 4, 32, ctypes.c_void_p(1 << 44),
                  None) == kvq.KVQ_ERR_UNSUPPORTED


def test_attend_f32_rejects_before_launch():
    assert lib.kvq_attend_f32(FAKE, FAKE, None, 1, 1, 1, 1, 8, 32, 0.0, 1, None, 0, FAKE2,
                              None) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_attend_f32(FAKE, FAKE, FAKE, 1, 1, 1, 1, 8, 96, 0.0, 1, None, 0, FAKE2,
                              None) == kvq.KVQ_ERR_UNSUPPORTED


def test_stream_read_rejects_bad_arguments():
    for data, nbytes, sink in ((None, 1024, FAKE2), (FAKE, 1024, None), (FAKE, 0, FAKE2),
                               (FAKE, 1000, FAKE2), (ctypes.c_void_p(0x10008), 1024, FAKE2)):
        assert lib.kvq_stream_read(data, nbytes, sink, None) == kvq.KVQ_ERR_INVALID



def _attend_cache(N, capacity, **kw):
    a = dict(q=FAKE, kc=FAKE, ks=FAKE, vc=FAKE, vs=FAKE, D=32, variant=0, out=FAKE2, flags=0, R=1)
    a.update(kw)
    return lib.kvq_attend_cache(a["q"], a["kc"], a["ks"], a["vc"], a["vs"], 1, 4, 2, a["R"], N,
                                capacity, a["D"], 4, 32, 0.0, 1, None, 0, a["out"], a["variant"],
                                a["flags"], None)


def test_attend_cache_rejects_before_launch():
    assert _attend_cache(64, 63) == kvq.KVQ_ERR_INVALID               # capacity < N
    assert _attend_cache(64, 64, q=None) == kvq.KVQ_ERR_INVALID
    assert _attend_cache(0, 64) == kvq.KVQ_ERR_INVALID
    # matrix-core limits apply to the capacity (the per-head buffer extent)
    assert _attend_cache(64, (1 << 25) - 31, D=128, variant=2,
                         out=ctypes.c_void_p(1 << 44)) == kvq.KVQ_ERR_UNSUPPORTED
    assert _attend_cache(64, 64, flags=2) == kvq.KVQ_ERR_INVALID      # unknown flag
    assert _attend_cache(64, 64, flags=-1) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_last_error()


def _append(**kw):
    a = dict(k=FAKE, v=FAKE, B=1, H=2, N=5, T=3, cap=16, D=8, bits=4, group=8,
             kc=ctypes.c_void_p(1 << 30), ks=ctypes.c_void_p(2 << 30), vc=ctypes.c_void_p(3 << 30),
             vs=ctypes.c_void_p(4 << 30), tail=ctypes.c_void_p(5 << 30))
    a.update(kw)
    return lib.kvq_append(a["k"], a["v"], a["B"], a["H"], a["N"], a["T"], a["cap"], a["D"],
                          a["bits"], a["group"], a["kc"], a["ks"], a["vc"], a["vs"], a["tail"],
                          None)


@pytest.mark.parametrize("kw", [
    dict(k=None), dict(tail=None), dict(vs=None),
    dict(T=0), dict(N=-1), dict(B=0), dict(D=0),
    dict(N=14, T=3),                                   # past the capacity
    dict(cap=0, N=0, T=1),
    dict(bits=6), dict(group=5),
    dict(k=ctypes.c_void_p(0x10002)),                  # misaligned float pointer
    dict(tail=ctypes.c_void_p((1 << 30) + 64)),        # tail inside the K codes
    dict(k=ctypes.c_void_p(3 << 30)),                  # new rows inside the V codes
])
def test_append_rejects_before_launch(kw):
    assert _append(**kw) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_last_error()


def test_cache_clear_rejects_before_launch():
    ptrs = [ctypes.c_void_p(i << 30) for i in (1, 2, 3, 4)]
    assert lib.kvq_cache_clear(1, 1, 0, 8, 4, 8, *ptrs, None) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_cache_clear(1, 1, 16, 8, 4, 9, *ptrs, None) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_cache_clear(1, 1, 16, 8, 4, 8, None, *ptrs[1:], None) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_cache_clear(1, 1, 16, 8, 4, 8, ptrs[0], ctypes.c_void_p((2 << 30) + 2),
                               *ptrs[2:], None) == kvq.KVQ_ERR_INVALID


def _attend_window(**kw):
    a = dict(q=FAKE, kw=ctypes.c_void_p(3 << 30), vw=ctypes.c_void_p(4 << 30), N=64, W=8,
             cap=64, flags=0, out=FAKE2)
    a.update(kw)
    return lib.kvq_attend_window(a["q"], FAKE, FAKE, FAKE, FAKE, a["kw"], a["vw"], 1, 4, 2, 1,
                                 a["N"], a["W"], a["cap"], 32, 4, 32, 0.0, 1, None, 0, a["out"],
                                 a["flags"], None)


@pytest.mark.parametrize("kw", [
    dict(kw=None), dict(vw=None), dict(W=0), dict(N=-1), dict(cap=63), dict(cap=0, N=0),
    dict(flags=4), dict(kw=ctypes.c_void_p((3 << 30) + 2)),
    dict(out=ctypes.c_void_p((4 << 30) + 64)),          # out inside the V window
])
def test_attend_window_rejects_before_launch(kw):
    assert _attend_window(**kw) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_last_error()


# --- size bounds that keep the 32-bit layout arithmetic from overflowing ---------------------

BIG_N = 0x7fffffff - (1 << 16) + 1     # one past the largest token count
BIG_D = (1 << 24) + 1                  # one past the largest head dimension


def test_sizes_reject_out_of_range():
    assert lib.kvq_k_code_bytes(1, 1, 128, 32, 4, 1 << 17) == 0           # group > 2^16
    assert lib.kvq_v_code_bytes(1, 1, 128, 32, 4, (1 << 16) + 2) == 0
    assert lib.kvq_k_code_bytes(1, 1, 128, 32, 4, 1 << 16) > 0            # group 2^16 is fine
    for fn in (lib.kvq_k_code_bytes, lib.kvq_k_scale_count, lib.kvq_v_code_bytes,
               lib.kvq_v_scale_count):
        assert fn(1, 1, BIG_N, 32, 4, 32) == 0
        assert fn(1, 1, 128, BIG_D, 4, 32) == 0
        assert fn(1, 1, BIG_N - 1, 8, 4, 32) > 0


def test_codec_and_cache_reject_out_of_range():
    for fn in (lib.kvq_pack_k, lib.kvq_pack_v):
        assert fn(FAKE, 1, 1, 8, 8, 4, 1 << 17, FAKE, FAKE2, None) == kvq.KVQ_ERR_INVALID
        assert fn(FAKE, 1, 1, BIG_N, 8, 4, 8, FAKE, FAKE2, None) == kvq.KVQ_ERR_INVALID
        assert fn(FAKE, 1, 1, 8, BIG_D, 4, 8, FAKE, FAKE2, None) == kvq.KVQ_ERR_INVALID
    for fn in (lib.kvq_dequant_k, lib.kvq_dequant_v):
        assert fn(FAKE, FAKE2, 1, 1, BIG_N, 8, 4, 8, ctypes.c_void_p(1 << 44),
                  None) == kvq.KVQ_ERR_INVALID
    ptrs = [ctypes.c_void_p(i << 30) for i in (1, 2, 3, 4)]
    assert lib.kvq_cache_clear(1, 1, BIG_N, 8, 4, 8, *ptrs, None) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_cache_clear(1, 1, 16, 8, 4, 1 << 17, *ptrs, None) == kvq.KVQ_ERR_INVALID
    assert _append(cap=BIG_N, N=BIG_N - 4) == kvq.KVQ_ERR_INVALID
    assert _append(group=1 << 17) == kvq.KVQ_ERR_INVALID


def test_attend_rejects_out_of_range():
    assert _attend(N=BIG_N) == kvq.KVQ_ERR_INVALID
    assert _attend(group=1 << 17) == kvq.KVQ_ERR_INVALID
    assert _attend_cache(64, BIG_N) == kvq.KVQ_ERR_INVALID
    assert _attend_window(N=BIG_N - 16, cap=BIG_N) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_last_error()


def test_study_rel_l2_closed_form():
    """The GPU study's per-input error is the page's ||O_q - O_f32||_F /
    ||O_f32||_F: on the hand-worked case (reference rows (3, 4, 0) and
    (0, 0, 12), one entry off by 5) it is 5/13, not a per-row mean (1/2)."""
    from quantized_kv_cache_attend_amd import accuracy
    ref = np.array([[3.0, 4.0, 0.0], [0.0, 0.0, 12.0]])
    approx = np.array([[3.0, 4.0, 5.0], [0.0, 0.0, 12.0]])
    assert accuracy.rel_l2(approx, ref) == pytest.approx(5.0 / 13.0, rel=1e-15)


def test_phase_trace_fetch_only_in_the_trace_build():
    """kvq_phase_trace_fetch is exported by every build; the normal library
    records nothing and says so before touching the device, and bad
    arguments are rejected first."""
    buf = (ctypes.c_uint64 * 16)()
    assert lib.kvq_phase_trace_fetch(0, ctypes.cast(buf, ctypes.c_void_p), 128) == kvq.KVQ_ERR_UNSUPPORTED
    assert lib.kvq_phase_trace_fetch(1, ctypes.cast(buf, ctypes.c_void_p), 128) == kvq.KVQ_ERR_UNSUPPORTED
    assert lib.kvq_phase_trace_fetch(2, ctypes.cast(buf, ctypes.c_void_p), 128) == kvq.KVQ_ERR_UNSUPPORTED
    assert lib.kvq_phase_trace_fetch(3, ctypes.cast(buf, ctypes.c_void_p), 128) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_phase_trace_fetch(-1, ctypes.cast(buf, ctypes.c_void_p), 128) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_phase_trace_fetch(0, None, 128) == kvq.KVQ_ERR_INVALID
    assert lib.kvq_phase_trace_fetch(0, ctypes.cast(buf, ctypes.c_void_p), 12) == kvq.KVQ_ERR_INVALID
