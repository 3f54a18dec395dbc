"""Python binding of ``libkvq.so``: packed 4/8-bit KV-cache attention on gfx950.

Argument marshalling only: every step of packing, decoding and attention
runs in the library's HIP kernels.  PyTorch supplies device memory and the
current stream.  The names follow the C ABI in ``include/kvq.h``.

Importing this package loads ``libkvq.so`` and raises ``ImportError`` if it
has not been built (``python -m quantized_kv_cache_attend_amd.build``); there
is no fallback path.

torch is imported first: PyTorch-ROCm ships its own HIP runtime, and loading
it before ``libkvq.so`` makes the library bind to that same runtime (both
carry the soname libamdhip64.so.7), so streams and device pointers from torch
are valid in the library's launches.  Loading the system runtime first would
put a second HIP runtime under torch.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the CDLL below)

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY names another build of the same library (the host-ASan build
# that a CPU test loads); by default the in-tree libkvq.so.
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(_PKG, "libkvq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -m quantized_kv_cache_attend_amd.build)")

lib = ctypes.CDLL(LIB_PATH)

_c_int, _c_float, _c_size, _c_vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

# (name, restype, argtypes) of every function in include/kvq.h.
_SIGNATURES = {
    "kvq_k_code_bytes": (_c_size, [_c_int] * 6),
    "kvq_k_scale_count": (_c_size, [_c_int] * 6),
    "kvq_v_code_bytes": (_c_size, [_c_int] * 6),
    "kvq_v_scale_count": (_c_size, [_c_int] * 6),
    "kvq_attend_auto_splits": (_c_int, [_c_int] * 3),
    "kvq_attend_workspace_bytes": (_c_size, [_c_int] * 7),
    "kvq_pack_k": (_c_int, [_c_vp] + [_c_int] * 6 + [_c_vp, _c_vp, _c_vp]),
    "kvq_pack_v": (_c_int, [_c_vp] + [_c_int] * 6 + [_c_vp, _c_vp, _c_vp]),
    "kvq_dequant_k": (_c_int, [_c_vp, _c_vp] + [_c_int] * 6 + [_c_vp, _c_vp]),
    "kvq_dequant_v": (_c_int, [_c_vp, _c_vp] + [_c_int] * 6 + [_c_vp, _c_vp]),
    "kvq_attend": (_c_int, [_c_vp] * 5 + [_c_int] * 8 + [_c_float, _c_int, _c_vp, _c_size,
                                                         _c_vp, _c_vp]),
    "kvq_attend_variant": (_c_int, [_c_vp] * 5 + [_c_int] * 8 + [_c_float, _c_int, _c_vp,
                                                                 _c_size, _c_vp, _c_int, _c_vp]),
    "kvq_attend_noalloc": (_c_int, [_c_vp] * 5 + [_c_int] * 8 + [_c_float, _c_int, _c_vp,
                                                                 _c_vp]),
    "kvq_cache_clear": (_c_int, [_c_int] * 6 + [_c_vp] * 5),
    "kvq_append": (_c_int, [_c_vp] * 2 + [_c_int] * 8 + [_c_vp] * 6),
    "kvq_append_attend": (_c_int, [_c_vp] * 3 + [_c_int] * 9 + [_c_vp] * 5 + [
        _c_float, _c_int, _c_vp, _c_size, _c_vp, _c_vp]),
    "kvq_attend_cache": (_c_int, [_c_vp] * 5 + [_c_int] * 9 + [_c_float, _c_int, _c_vp, _c_size,
                                                               _c_vp, _c_int, _c_int, _c_vp]),
    "kvq_attend_window": (_c_int, [_c_vp] * 7 + [_c_int] * 10 + [_c_float, _c_int, _c_vp,
                                                                _c_size, _c_vp, _c_int, _c_vp]),
    "kvq_attend_f32": (_c_int, [_c_vp] * 3 + [_c_int] * 6 + [_c_float, _c_int, _c_vp, _c_size,
                                                             _c_vp, _c_vp]),
    "kvq_stream_read": (_c_int, [_c_vp, _c_size, _c_vp, _c_vp]),
    "kvq_phase_trace_fetch": (_c_int, [_c_int, _c_vp, _c_size]),
    "kvq_status_string": (ctypes.c_char_p, [_c_int]),
    "kvq_last_error": (ctypes.c_char_p, []),
    "kvq_abi_version": (_c_int, []),
}
for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

KVQ_OK, KVQ_ERR_INVALID, KVQ_ERR_UNSUPPORTED, KVQ_ERR_HIP, KVQ_ERR_WORKSPACE = 0, -1, -2, -3, -4
VARIANTS = {"auto": 0, "valu": 1, "mfma": 2, "stream": 3}
KVQ_ATTEND_CAUSAL = 1


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.kvq_last_error().decode() or lib.kvq_status_string(status).decode()
        super().__init__(f"{where}: {lib.kvq_status_string(status).decode()} ({status}): {msg}")


def _check(status: int, where: str) -> None:
    if status != KVQ_OK:
        raise KvqError(status, where)


def _torch():
    import torch
    return torch


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# --- sizing -------------------------------------------------------------------------

def packed_shapes(B, H, N, D, bits, group):
    """Shapes of (k_codes, k_scales, v_codes, v_scales) for K/V of [B,H,N,D]
    in the 32-token block layout of include/kvq.h."""
    nblocks = -(-N // 32)
    d8 = -(-D // 8)
    dpad = -(-D // group) * group
    return ((B, H, nblocks, d8 * 8 * 32 * bits // 8), (B, H, -(-N // group), D),
            (B, H, nblocks, 32 * dpad * bits // 8), (B, H, nblocks, dpad // group * 32))


def workspace_bytes(B, Hq, Hkv, R, N, D, num_splits=0) -> int:
    return int(lib.kvq_attend_workspace_bytes(B, Hq, Hkv, R, N, D, num_splits))


def auto_splits(B, Hkv, N) -> int:
    return int(lib.kvq_attend_auto_splits(B, Hkv, N))


def new_workspace(B, Hq, Hkv, R, N, D, num_splits=0, device="cuda"):
    """A zero-filled workspace (the library requires zeros before first use)."""
    torch = _torch()
    n = workspace_bytes(B, Hq, Hkv, R, N, D, num_splits)
    ws = torch.zeros(n, dtype=torch.uint8, device=device)
    ws._kvq_clean = n  # every byte is zero: any call's counters start at 0
    return ws


# Bytes between two arrival counters at the start of a workspace (one counter
# per (batch, KV head); include/kvq.h, kvq_attend_workspace_bytes).
_COUNTER_STRIDE = 256


def _prepare_workspace(ws, heads, name="workspace"):
    """Check a caller's workspace and return its size in bytes.  The library
    keeps one arrival counter per (batch, KV head) at the start of the
    workspace and needs them zero when a call starts; every completed call
    leaves its own counters zero and may write split partials right after
    them.  So after a call on `heads` pairs only the first 256 * heads bytes
    are known to be zero: a later call on more pairs would find partials where
    its extra counters go, and that range is zero-filled here (a fill kernel
    on the current stream) before it runs.  A workspace this binding has not
    seen before is taken to be zero-filled, as the C contract requires."""
    torch = _torch()
    if not isinstance(ws, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not ws.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    nbytes = ws.numel() * ws.element_size()
    need = min(_COUNTER_STRIDE * heads, nbytes)
    clean = getattr(ws, "_kvq_clean", need)
    if clean < need:
        ws.view(torch.uint8)[clean:need].zero_()
    ws._kvq_clean = need  # what the call leaves known-zero (its partials follow)
    return nbytes


def _check_out(out, shape, device):
    torch = _torch()
    _need(out, torch.float32, "out")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must have shape {tuple(shape)}, got {tuple(out.shape)}")
    if out.device != device:
        raise ValueError("out must be on the same device as q")


# --- calls -----------------------------------------------------------------------------

def _pack(fn, x, bits, group, k_style):
    torch = _torch()
    _need(x, torch.float32, "x")
    B, H, N, D = x.shape
    ks, kss, vs, vss = packed_shapes(B, H, N, D, bits, group)
    cshape, sshape = (ks, kss) if k_style else (vs, vss)
    codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(sshape, dtype=torch.float32, device=x.device)
    _check(fn(_ptr(x), B, H, N, D, bits, group, _ptr(codes), _ptr(scales), _stream(x.device)),
           fn.__name__)
    return codes, scales


def pack_k(k, bits=4, group=32):
    """Pack float32 K [B,H,N,D] -> (codes u8, scales f32) in the block layout."""
    return _pack(lib.kvq_pack_k, k, bits, group, True)


def pack_v(v, bits=4, group=32):
    """Pack float32 V [B,H,N,D] -> (codes u8, scales f32) in the block layout."""
    return _pack(lib.kvq_pack_v, v, bits, group, False)


def _dequant(fn, codes, scales, N, D, bits, group, out):
    torch = _torch()
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.float32, "scales")
    B, H = codes.shape[:2]
    if out is None:
        out = torch.empty((B, H, N, D), dtype=torch.float32, device=codes.device)
    _need(out, torch.float32, "out")
    if tuple(out.shape) != (B, H, N, D):
        raise ValueError(f"out must have shape {(B, H, N, D)}")
    _check(fn(_ptr(codes), _ptr(scales), B, H, N, D, bits, group, _ptr(out),
              _stream(codes.device)), fn.__name__)
    return out


def dequant_k(codes, scales, N, D, bits=4, group=32, out=None):
    """Decode packed K to float32 [B,H,N,D]."""
    return _dequant(lib.kvq_dequant_k, codes, scales, N, D, bits, group, out)


def dequant_v(codes, scales, N, D, bits=4, group=32, out=None):
    """Decode packed V to float32 [B,H,N,D]."""
    return _dequant(lib.kvq_dequant_v, codes, scales, N, D, bits, group, out)


def _check_cache(arrays, B, H, cap, D, bits, group):
    """The four packed arrays hold at least the layout's elements for `cap` tokens."""
    for t, shape, name in zip(arrays, packed_shapes(B, H, cap, D, bits, group),
                              ("k_codes", "k_scales", "v_codes", "v_scales")):
        need = 1
        for n in shape:
            need *= n
        if t.numel() < need:
            raise ValueError(f"{name} holds {t.numel()} elements, the layout for {cap} tokens "
                             f"needs {need}")


def attend(q, k_codes, k_scales, v_codes, v_scales, N, bits=4, group=32, sm_scale=0.0,
           num_splits=0, workspace=None, out=None, variant="auto", capacity=None, causal=False):
    """Fused attention of q [B,Hq,R,D] over the first N tokens of the packed
    cache (KV heads = k_codes.shape[1]); `capacity`: the tokens the cache
    layout is sized for (default N; a cache grown by append()); `causal`: the
    R queries are the last R positions and read only tokens up to their own."""
    torch = _torch()
    _need(q, torch.float32, "q")
    for t, n, dt in ((k_codes, "k_codes", torch.uint8), (k_scales, "k_scales", torch.float32),
                     (v_codes, "v_codes", torch.uint8), (v_scales, "v_scales", torch.float32)):
        _need(t, dt, n)
    B, Hq, R, D = q.shape
    Hkv = k_codes.shape[1]
    cap = N if capacity is None else capacity
    if bits in (4, 8) and group >= 2 and N >= 1 and cap >= N:
        _check_cache((k_codes, k_scales, v_codes, v_scales), B, Hkv, cap, D, bits, group)
    if workspace is None:
        workspace = new_workspace(B, Hq, Hkv, R, N, D, num_splits, device=q.device)
    ws_bytes = _prepare_workspace(workspace, B * Hkv)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q.shape, q.device)
    if variant not in VARIANTS:
        raise ValueError(f"variant must be one of {sorted(VARIANTS)}")
    if capacity is None and not causal:
        _check(lib.kvq_attend_variant(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                                      _ptr(v_scales), B, Hq, Hkv, R, N, D, bits, group,
                                      float(sm_scale), num_splits, _ptr(workspace), ws_bytes,
                                      _ptr(out), VARIANTS[variant], _stream(q.device)),
               "kvq_attend")
    else:
        _check(lib.kvq_attend_cache(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                                    _ptr(v_scales), B, Hq, Hkv, R, N, cap, D, bits, group,
                                    float(sm_scale), num_splits, _ptr(workspace), ws_bytes,
                                    _ptr(out), VARIANTS[variant],
                                    KVQ_ATTEND_CAUSAL if causal else 0, _stream(q.device)),
               "kvq_attend_cache")
    return out


def attend_noalloc(q, k_codes, k_scales, v_codes, v_scales, N, bits=4, group=32, sm_scale=0.0,
                   num_splits=0, out=None):
    """kvq_attend_noalloc: kvq_attend with the library's own scratch as the
    workspace (no workspace argument, nothing allocated by the call when `out`
    is given)."""
    torch = _torch()
    _need(q, torch.float32, "q")
    for t, n, dt in ((k_codes, "k_codes", torch.uint8), (k_scales, "k_scales", torch.float32),
                     (v_codes, "v_codes", torch.uint8), (v_scales, "v_scales", torch.float32)):
        _need(t, dt, n)
    B, Hq, R, D = q.shape
    Hkv = k_codes.shape[1]
    if bits in (4, 8) and group >= 2 and N >= 1:
        _check_cache((k_codes, k_scales, v_codes, v_scales), B, Hkv, N, D, bits, group)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q.shape, q.device)
    _check(lib.kvq_attend_noalloc(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                                  _ptr(v_scales), B, Hq, Hkv, R, N, D, bits, group,
                                  float(sm_scale), num_splits, _ptr(out), _stream(q.device)),
           "kvq_attend_noalloc")
    return out


def attend_window(q, k_codes, k_scales, v_codes, v_scales, k_win, v_win, N, bits=4, group=32,
                  capacity=None, sm_scale=0.0, num_splits=0, workspace=None, out=None,
                  causal=False):
    """Attention over N packed tokens followed by the W = k_win.shape[2]
    most recent tokens in float32 (k_win, v_win [B,Hkv,W,D])."""
    torch = _torch()
    _need(q, torch.float32, "q")
    for t, n, dt in ((k_codes, "k_codes", torch.uint8), (k_scales, "k_scales", torch.float32),
                     (v_codes, "v_codes", torch.uint8), (v_scales, "v_scales", torch.float32),
                     (k_win, "k_win", torch.float32), (v_win, "v_win", torch.float32)):
        _need(t, dt, n)
    B, Hq, R, D = q.shape
    Hkv, W = k_win.shape[1], k_win.shape[2]
    if tuple(k_win.shape) != (B, Hkv, W, D) or k_win.shape != v_win.shape:
        raise ValueError("k_win and v_win must both be [B, Hkv, W, D]")
    cap = max(N, 1) if capacity is None else capacity
    if bits in (4, 8) and group >= 2 and cap >= max(N, 1):
        _check_cache((k_codes, k_scales, v_codes, v_scales), B, Hkv, cap, D, bits, group)
    if workspace is None:  # a slot per 32 window tokens beyond the splits: the fused form
        slots = (num_splits or auto_splits(B, Hkv, N + W)) + (W + 31) // 32
        workspace = new_workspace(B, Hq, Hkv, R, N + W, D, slots, device=q.device)
    ws_bytes = _prepare_workspace(workspace, B * Hkv)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q.shape, q.device)
    _check(lib.kvq_attend_window(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                                 _ptr(v_scales), _ptr(k_win), _ptr(v_win), B, Hq, Hkv, R, N, W,
                                 cap, D, bits, group, float(sm_scale), num_splits,
                                 _ptr(workspace), ws_bytes, _ptr(out),
                                 KVQ_ATTEND_CAUSAL if causal else 0, _stream(q.device)),
           "kvq_attend_window")
    return out


# --- growing cache (decode steps) -------------------------------------------------------

def new_cache(B, H, capacity, D, bits=4, group=32, device="cuda"):
    """An empty packed cache for `capacity` tokens (kvq_cache_clear) and its
    float32 K tail: (k_codes, k_scales, v_codes, v_scales, k_tail)."""
    torch = _torch()
    kcs, kss, vcs, vss = packed_shapes(B, H, capacity, D, bits, group)
    kc = torch.empty(kcs, dtype=torch.uint8, device=device)
    ks = torch.empty(kss, dtype=torch.float32, device=device)
    vc = torch.empty(vcs, dtype=torch.uint8, device=device)
    vs = torch.empty(vss, dtype=torch.float32, device=device)
    tail = torch.zeros((B, H, group, D), dtype=torch.float32, device=device)
    _check(lib.kvq_cache_clear(B, H, capacity, D, bits, group, _ptr(kc), _ptr(ks), _ptr(vc),
                               _ptr(vs), _stream(kc.device)), "kvq_cache_clear")
    return kc, ks, vc, vs, tail


def append(k_new, v_new, N, cache, capacity, bits=4, group=32):
    """Append k_new, v_new [B,H,T,D] float32 after the first N tokens of
    `cache` (the tuple new_cache returns) laid out for `capacity` tokens."""
    torch = _torch()
    _need(k_new, torch.float32, "k_new")
    _need(v_new, torch.float32, "v_new")
    if k_new.shape != v_new.shape or k_new.dim() != 4:
        raise ValueError("k_new and v_new must both be [B, H, T, D]")
    kc, ks, vc, vs, tail = cache
    for t, n, dt in ((kc, "k_codes", torch.uint8), (ks, "k_scales", torch.float32),
                     (vc, "v_codes", torch.uint8), (vs, "v_scales", torch.float32),
                     (tail, "k_tail", torch.float32)):
        _need(t, dt, n)
    B, H, T, D = k_new.shape
    if bits in (4, 8) and group >= 2 and capacity >= 1:
        _check_cache((kc, ks, vc, vs), B, H, capacity, D, bits, group)
        if tail.numel() < B * H * group * D:
            raise ValueError(f"k_tail must hold [B, H, group, D] = {(B, H, group, D)}")
    _check(lib.kvq_append(_ptr(k_new), _ptr(v_new), B, H, N, T, capacity, D, bits, group,
                          _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs), _ptr(tail),
                          _stream(k_new.device)), "kvq_append")


def append_attend(q, k_new, v_new, N, cache, capacity, bits=4, group=32, sm_scale=0.0,
                  num_splits=0, workspace=None, out=None):
    """One decode step (kvq_append_attend): append k_new, v_new [B,Hkv,1,D]
    float32 after the first N tokens of `cache` (the tuple new_cache returns,
    laid out for `capacity` tokens), then attend q [B,Hq,R,D] over the N + 1
    tokens.  Same bytes and output as append() followed by attend(...,
    capacity=capacity); one launch when the 4-row matrix-core kernel serves
    the step."""
    torch = _torch()
    _need(q, torch.float32, "q")
    _need(k_new, torch.float32, "k_new")
    _need(v_new, torch.float32, "v_new")
    kc, ks, vc, vs, tail = cache
    for t, n, dt in ((kc, "k_codes", torch.uint8), (ks, "k_scales", torch.float32),
                     (vc, "v_codes", torch.uint8), (vs, "v_scales", torch.float32),
                     (tail, "k_tail", torch.float32)):
        _need(t, dt, n)
    B, Hq, R, D = q.shape
    Hkv = kc.shape[1]
    if tuple(k_new.shape) != (B, Hkv, 1, D) or tuple(v_new.shape) != (B, Hkv, 1, D):
        raise ValueError(f"k_new and v_new must both be [B, Hkv, 1, D] = {(B, Hkv, 1, D)}")
    if bits in (4, 8) and group >= 2 and capacity >= 1:
        _check_cache((kc, ks, vc, vs), B, Hkv, capacity, D, bits, group)
        if tail.numel() < B * Hkv * group * D:
            raise ValueError(f"k_tail must hold [B, H, group, D] = {(B, Hkv, group, D)}")
    if workspace is None:
        workspace = new_workspace(B, Hq, Hkv, R, N + 1, D, num_splits, device=q.device)
    ws_bytes = _prepare_workspace(workspace, B * Hkv)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q.shape, q.device)
    _check(lib.kvq_append_attend(_ptr(q), _ptr(k_new), _ptr(v_new), B, Hq, Hkv, R, N, capacity,
                                 D, bits, group, _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs),
                                 _ptr(tail), float(sm_scale), num_splits, _ptr(workspace),
                                 ws_bytes, _ptr(out), _stream(q.device)), "kvq_append_attend")
    return out


def attend_f32(q, k, v, sm_scale=0.0, num_splits=0, workspace=None, out=None):
    """Attention of q [B,Hq,R,D] over a float32 cache k, v [B,Hkv,N,D]."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.float32, n)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, Hq, R, D] and k, v [B, Hkv, N, D]")
    B, Hq, R, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v must have k's shape {tuple(k.shape)}, got {tuple(v.shape)}")
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k must be [B={B}, Hkv, N, D={D}], got {tuple(k.shape)}")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on one device")
    if workspace is None:
        workspace = new_workspace(B, Hq, Hkv, R, N, D, num_splits, device=q.device)
    ws_bytes = _prepare_workspace(workspace, B * Hkv)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q.shape, q.device)
    _check(lib.kvq_attend_f32(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, R, N, D, float(sm_scale),
                              num_splits, _ptr(workspace), ws_bytes, _ptr(out),
                              _stream(q.device)), "kvq_attend_f32")
    return out


def stream_read(data, sink=None):
    """Read every byte of the device tensor `data` once (kvq_stream_read): the
    plain streaming-read ceiling the fused attend is measured against.
    `sink` (a one-word int32 device tensor, allocated if omitted) is written
    only if the XOR of the data equals an arbitrary constant."""
    torch = _torch()
    if not data.is_cuda or not data.is_contiguous():
        raise ValueError("stream_read needs a contiguous device tensor")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=data.device)
    nbytes = data.numel() * data.element_size()
    _check(lib.kvq_stream_read(_ptr(data), nbytes, _ptr(sink), _stream(data.device)),
           "kvq_stream_read")
    return sink
