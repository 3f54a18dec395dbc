"""Plain float64 CPU oracle for attention over a packed 4/8-bit KV cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
of ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or run this module.  It shares no code, table or constant generator with the
HIP library: it imports nothing but NumPy and the standard library, and the
library never imports it.

Every function follows a passage of the pages that describe the method.  The
pages are cited by title, with the section (or table / formula block) that a
step follows:

  [BKD]  "Block KV decoding: less workspace, more time"
         (huhohoo.com/en/docs/llm/kv-block-decode-cost; the Chinese twin is
         "KV分块反量化：工作区小了，为什么更慢？")
  [KPG]  "KV分组打包：4-bit到底省了多少？" (huhohoo.com/docs/llm/kv-packed-groups)
  [TOS]  "注意力分塊：不保存完整分數矩陣，如何保持結果？"
         (huhohoo.com/zh-TW/docs/llm/tiled-online-softmax)
  [RL]   "给长前缀列一张有单位的资源账本"
         (codingai-lec05.pages.dev, resource-ledger)

Precision.  The pages fix the quantizer's storage types (uint8 codes, float32
scales, [KPG] "what a byte holds"), decode into float32 arrays ([BKD] "Which
arrays shrink?") and then run all attention arithmetic in float64 ([BKD]
"Compare equivalent representations first").  The quantizer's own arithmetic
(max|x|/7, x/scale, rint) is therefore done in IEEE float32 with NumPy's
float32 semantics (correctly rounded division, round-half-to-even), and every
step after the float32 decode is float64.

Parity status of each function is stated in its docstring; the pins live in
``tests/test_oracle_*.py`` and ``tests/golden/``.
"""
from __future__ import annotations

import math

import numpy as np

# Largest code magnitude per bit width: [-7, 7] for 4-bit, [-127, 127] for
# 8-bit ([KPG] "what a byte holds").
QMAX = {4: 7, 8: 127}


def _check_format(bits: int, group: int) -> None:
    if bits not in QMAX:
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    if group < 2 or group % 2:
        raise ValueError(f"group must be even and >= 2, got {group}")


# ---------------------------------------------------------------------------
# Grouping, quantization, nibble packing
# ---------------------------------------------------------------------------

def group_last(x: np.ndarray, axis: int, group: int) -> np.ndarray:
    """Move ``axis`` last, zero-pad it to a multiple of ``group`` and split it
    into ``[..., L/group, group]``.

    [KPG] "why grouping needs both direction and length": K is grouped along
    tokens inside each channel, V along features inside each token; a short
    final group is padded with zeros and cropped again on decode.
    """
    y = np.moveaxis(np.asarray(x), axis, -1)
    length = y.shape[-1]
    padded = -(-length // group) * group
    if padded != length:
        widths = [(0, 0)] * (y.ndim - 1) + [(0, padded - length)]
        y = np.pad(y, widths)
    return y.reshape(y.shape[:-1] + (padded // group, group))


def quantize_groups(groups: np.ndarray, bits: int):
    """Symmetric per-group quantization of a ``[..., G, g]`` float32 array.

    Returns ``(stored, scales)``: ``stored`` uint8 codes offset by +7 (+127),
    ``scales`` float32 of shape ``[..., G]``.

    [KPG] "what a byte holds": scale = max(abs(x))/7, codes in [-7, 7], stored
    +7 so they sit in [0, 14] (15 unused); the 8-bit variant uses 127.
    [KPG] "exercises and common mistakes": an all-zero group takes scale 1.
    Readings where the page is silent: codes are round-half-to-even of the
    float32 quotient, then clipped; the scale fallback applies whenever the
    float32 scale is exactly 0 (an all-zero group, or max|x| so small that
    max|x|/7 underflows to 0).
    """
    y = np.asarray(groups, dtype=np.float32)
    qmax = np.float32(QMAX[bits])
    scales = (np.max(np.abs(y), axis=-1) / qmax).astype(np.float32)
    scales = np.where(scales == np.float32(0.0), np.float32(1.0), scales).astype(np.float32)
    quotient = (y / scales[..., None]).astype(np.float32)
    codes = np.clip(np.rint(quotient), -qmax, qmax)
    stored = (codes + qmax).astype(np.uint8)
    return stored, scales


def pack_nibbles(stored: np.ndarray) -> np.ndarray:
    """Pack a flat stream of 4-bit stored codes two per byte.

    [KPG] "what a byte holds": element 2i goes to the low nibble and element
    2i+1 to the high nibble of byte i.  The stream is the grouped array
    flattened in C order; groups have even length, so no byte straddles two
    groups or two rows.
    """
    flat = np.ascontiguousarray(stored, dtype=np.uint8).reshape(-1)
    if flat.size % 2:
        raise ValueError("nibble packing needs an even number of codes")
    return (flat[0::2] | (flat[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_nibbles`: ``&15`` gives the even element, ``>>4``
    the odd one ([KPG] "what a byte holds")."""
    flat = np.ascontiguousarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(flat.size * 2, dtype=np.uint8)
    out[0::2] = flat & 15
    out[1::2] = flat >> 4
    return out


def pack(x: np.ndarray, axis: int, bits: int, group: int):
    """Quantize and pack ``x`` with groups running along ``axis``.

    Returns ``(codes, scales)`` where, with ``L`` the grouped axis padded to a
    multiple of ``group`` and the grouped axis moved last,
    ``codes`` has shape ``[..., L*bits/8]`` (uint8) and ``scales`` has shape
    ``[..., L/group]`` (float32).  For K of shape ``[B, H, N, D]`` and
    ``axis=-2`` that is codes ``[B, H, D, Npad*bits/8]`` and scales
    ``[B, H, D, Npad/group]``; for V with ``axis=-1`` it is codes
    ``[B, H, N, Dpad*bits/8]`` and scales ``[B, H, N, Dpad/group]``.

    Follows [KPG] "what a byte holds" and "why grouping needs both direction
    and length".
    """
    _check_format(bits, group)
    x = np.asarray(x, dtype=np.float32)
    grouped = group_last(x, axis, group)
    stored, scales = quantize_groups(grouped, bits)
    lead = grouped.shape[:-2]
    padded = grouped.shape[-2] * group
    if bits == 4:
        codes = pack_nibbles(stored).reshape(lead + (padded // 2,))
    else:
        codes = stored.reshape(lead + (padded,))
    return codes, scales


def unpack_stored(codes: np.ndarray, shape, axis: int, bits: int, group: int) -> np.ndarray:
    """Recover the stored (offset) codes in the original layout of ``shape``.

    [KPG] "what a byte holds" and "exercises and common mistakes": unpack the
    nibbles, regroup, crop the padding off the grouped axis, then move the
    axis back, so a non-divisible shape gains no extra row or column.
    """
    _check_format(bits, group)
    shape = tuple(shape)
    nd = len(shape)
    ax = axis % nd
    length = shape[ax]
    padded = -(-length // group) * group
    moved = tuple(s for i, s in enumerate(shape) if i != ax)
    if bits == 4:
        stored = unpack_nibbles(codes)
    else:
        stored = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    stored = stored.reshape(moved + (padded,))[..., :length]
    return np.moveaxis(stored, -1, ax)


def expand_scales(scales: np.ndarray, shape, axis: int, group: int) -> np.ndarray:
    """Broadcast per-group scales back onto every element of ``shape`` (crop
    the padded tail, restore the axis)."""
    shape = tuple(shape)
    ax = axis % len(shape)
    length = shape[ax]
    per_element = np.repeat(np.asarray(scales, dtype=np.float32), group, axis=-1)[..., :length]
    return np.moveaxis(per_element, -1, ax)


def dequant(codes: np.ndarray, scales: np.ndarray, shape, axis: int, bits: int,
            group: int) -> np.ndarray:
    """Decode a packed array to float32: ``fl32((stored - qmax) * scale)``.

    [KPG] "what a byte holds": subtract the offset and multiply by the group's
    scale; the pages decode into float32 arrays ([BKD] "Which arrays shrink?").
    The integer ``stored - qmax`` is exact in float32, so the result takes one
    float32 rounding, in the multiply.
    """
    stored = unpack_stored(codes, shape, axis, bits, group)
    centred = stored.astype(np.float32) - np.float32(QMAX[bits])
    return (centred * expand_scales(scales, shape, axis, group)).astype(np.float32)


def pack_k(k: np.ndarray, bits: int, group: int):
    """K-style packing of ``[..., N, D]``: groups of tokens inside each
    channel ([KPG] "why grouping needs both direction and length")."""
    return pack(k, -2, bits, group)


def pack_v(v: np.ndarray, bits: int, group: int):
    """V-style packing of ``[..., N, D]``: groups of features inside each
    token ([KPG] "why grouping needs both direction and length")."""
    return pack(v, -1, bits, group)


def dequant_k(codes, scales, shape, bits, group):
    return dequant(codes, scales, shape, -2, bits, group)


def dequant_v(codes, scales, shape, bits, group):
    return dequant(codes, scales, shape, -1, bits, group)


# ---------------------------------------------------------------------------
# Byte order in device memory
# ---------------------------------------------------------------------------
#
# The pages fix the groups, the scales and what one byte holds ([KPG] "what a
# byte holds": two neighbouring codes of one group, the lower-indexed one in
# the low nibble) but not the order of the bytes.  The library stores the
# cache in 32-token blocks (the byte order documented in include/kvq.h); the
# two functions below state that order with NumPy reshapes, starting from the
# canonical arrays above, so device packing can be compared byte for byte.
# Positions that hold no element store the zero code QMAX; V scales of
# tokens past N are 1, the scale of an all-zero group ([KPG] "exercises and
# common mistakes").

BLOCK_TOKENS = 32


def store_k(codes: np.ndarray, scales: np.ndarray, n: int, d: int, bits: int, group: int):
    """Canonical packed K (``pack_k``) -> block layout.

    Codes become ``[..., nblocks, D8*kcols*8]``: inside a block the byte
    ``(o*kcols + j)*8 + e`` holds channel ``8o+e`` of byte column ``j``, a
    4-bit column ``j`` pairing tokens ``2j`` (low nibble) and ``2j+1``
    (high), an 8-bit column ``j`` being token ``j``.  Scales become
    group-major ``[..., ceil(N/group), D]``.
    """
    _check_format(bits, group)
    lead = codes.shape[:-2]
    stored = unpack_stored(codes, lead + (n, d), -2, bits, group)      # [..., N, D]
    nb, d8 = -(-n // BLOCK_TOKENS), -(-d // 8)
    full = np.full(lead + (nb * BLOCK_TOKENS, d8 * 8), QMAX[bits], np.uint8)
    full[..., :n, :d] = stored
    tok = full.reshape(lead + (nb, BLOCK_TOKENS, d8, 8))                # [..., blk, t, o, e]
    if bits == 4:
        pairs = tok.reshape(lead + (nb, BLOCK_TOKENS // 2, 2, d8, 8))
        cols = pairs[..., 0, :, :] | (pairs[..., 1, :, :] << 4)         # [..., blk, j, o, e]
    else:
        cols = tok
    blocks = np.moveaxis(cols, -2, -3)                                  # [..., blk, o, j, e]
    k_store = np.ascontiguousarray(blocks).reshape(lead + (nb, -1))
    s_store = np.ascontiguousarray(np.swapaxes(np.asarray(scales, np.float32), -1, -2))
    return k_store, s_store


def store_v(codes: np.ndarray, scales: np.ndarray, n: int, d: int, bits: int, group: int):
    """Canonical packed V (``pack_v``) -> block layout.

    Codes become ``[..., nblocks, 4*vcols*8]``: inside a block the byte
    ``(o*vcols + f)*8 + e`` holds token ``8o+e`` of byte column ``f``, a
    4-bit column ``f`` pairing features ``2f`` (low) and ``2f+1`` (high).
    Scales become ``[..., nblocks, Dpad/group * 32]``, token-minor.
    """
    _check_format(bits, group)
    lead = codes.shape[:-2]
    stored = unpack_stored(codes, lead + (n, d), -1, bits, group)      # [..., N, D]
    nb = -(-n // BLOCK_TOKENS)
    dpad = -(-d // group) * group
    full = np.full(lead + (nb * BLOCK_TOKENS, dpad), QMAX[bits], np.uint8)
    full[..., :n, :d] = stored
    tok = full.reshape(lead + (nb, 4, 8, dpad))                         # [..., blk, o, e, f]
    if bits == 4:
        pairs = tok.reshape(lead + (nb, 4, 8, dpad // 2, 2))
        cols = pairs[..., 0] | (pairs[..., 1] << 4)                     # [..., blk, o, e, col]
    else:
        cols = tok
    blocks = np.swapaxes(cols, -1, -2)                                  # [..., blk, o, col, e]
    v_store = np.ascontiguousarray(blocks).reshape(lead + (nb, -1))
    sc = np.asarray(scales, np.float32)
    padded = np.ones(lead + (nb * BLOCK_TOKENS, sc.shape[-1]), np.float32)
    padded[..., :n, :] = sc
    per_block = padded.reshape(lead + (nb, BLOCK_TOKENS, sc.shape[-1]))
    s_store = np.ascontiguousarray(np.swapaxes(per_block, -1, -2)).reshape(lead + (nb, -1))
    return v_store, s_store


# ---------------------------------------------------------------------------
# A cache that grows by decode steps
# ---------------------------------------------------------------------------

def cache_after(k: np.ndarray, v: np.ndarray, n: int, capacity: int, bits: int, group: int):
    """The packed cache, in the block layout for ``capacity`` tokens, once the
    first ``n`` tokens of K and V ``[..., N, D]`` have been appended to it.

    [RL] "prefill and decode": a decode step reads the cached K/V and appends
    its new position.  Reading: the cache of n tokens is the packed tensor of
    those n tokens ([KPG] "what a byte holds"), its short groups zero-padded
    ([KPG] "why grouping needs both direction and length"), laid out for the
    capacity; positions past n are zeros before quantization, so they hold
    the zero code with scale 1 where a whole group is empty.
    Parity: pinned in tests/test_oracle_cache.py (equality with plain packing
    at n = capacity; the byte formula of the layout read back independently;
    a token-by-token append that requantizes the open K group).
    """
    _check_format(bits, group)
    lead, d = k.shape[:-2], k.shape[-1]
    kp = np.zeros(lead + (capacity, d), np.float32)
    vp = np.zeros(lead + (capacity, d), np.float32)
    kp[..., :n, :] = k[..., :n, :]
    vp[..., :n, :] = v[..., :n, :]
    kc, ks = store_k(*pack_k(kp, bits, group), capacity, d, bits, group)
    vc, vs = store_v(*pack_v(vp, bits, group), capacity, d, bits, group)
    return kc, ks, vc, vs


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _gqa_rows(q: np.ndarray, hkv: int) -> np.ndarray:
    """View ``q [B, Hq, R, D]`` as ``[B, Hkv, (Hq/Hkv)*R, D]``.

    [RL] "GQA changes the shared interface": each group of Hq/Hkv query heads
    reads one K/V head.  Reading: the map is contiguous, query head ``h``
    reads KV head ``h // (Hq/Hkv)``.
    """
    b, hq, r, d = q.shape
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return q.reshape(b, hkv, (hq // hkv) * r, d)


def default_scale(d: int) -> float:
    """Softmax temperature ``1/sqrt(d)``: [RL] "prefill and decode" writes the
    scores as ``S = Q K^T / sqrt(d_k)``."""
    return 1.0 / math.sqrt(d)


def causal_mask(n: int, r: int) -> np.ndarray:
    """Which of ``n`` cached tokens each of ``r`` queries may read when the
    queries are the sequence's last ``r`` positions (a prefill chunk or a
    multi-token decode step): query ``i`` sits at position ``n - r + i`` and
    reads token ``j`` iff ``j <= n - r + i``.  ``[r, n]`` bool.

    [RL] "prefill and decode" (a causal kernel reads only the keys at or
    before each query) and [TOS] opening section (its queries read every
    position, which does not stand in for a causal prefill).  Reading: the
    chunk is aligned to the end of the cache; when ``n < r`` the first
    ``r - n`` queries read nothing.
    """
    return np.arange(n)[None, :] <= (n - r + np.arange(r))[:, None]


def attend_dense(q, k_hat, v_hat, sm_scale=None, trace=None, causal=False):
    """Dense ``softmax(Q K^T * sm_scale) V`` in float64.

    ``q`` is ``[B, Hq, R, D]``; ``k_hat``/``v_hat`` are ``[B, Hkv, N, D]``
    (decoded float32 or raw float32, promoted to float64).  Returns
    ``[B, Hq, R, D]`` float64.

    This is the plain definition the blocked method must reproduce exactly up
    to rounding order: [BKD] "Compare equivalent representations first" (the
    dense decode-all path) and [RL] "why FlashAttention need not keep the whole
    heat map" (the row output is sum_j exp(s_j) v_j / sum_j exp(s_j), shifted
    by the max for stability).  No mask by default: the queries read every
    KV position ([TOS] opening section).  ``causal``: query ``i`` of the R
    per head reads only the tokens ``causal_mask`` allows; masked positions
    enter neither the max nor the sum, and a row with no legal key returns
    zeros ([RL] "why FlashAttention need not keep the whole heat map": such a
    row is handled explicitly, never as NaN).

    ``trace`` (optional dict) receives the byte sizes of the named work arrays
    ([BKD] "Which arrays shrink?").
    """
    d = q.shape[-1]
    scale = default_scale(d) if sm_scale is None else float(sm_scale)
    k64 = np.asarray(k_hat, dtype=np.float64)
    v64 = np.asarray(v_hat, dtype=np.float64)
    rows = _gqa_rows(np.asarray(q, dtype=np.float64), k64.shape[1])
    scores = np.matmul(rows, np.swapaxes(k64, -1, -2)) * scale
    if causal:
        r = q.shape[2]
        visible = np.tile(causal_mask(k64.shape[2], r), (rows.shape[2] // r, 1))
        scores = np.where(visible, scores, -np.inf)
    mx = scores.max(axis=-1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)          # rows with no legal key
    weights = np.exp(scores - mx)
    den = weights.sum(axis=-1, keepdims=True)
    out = np.matmul(weights, v64) / np.where(den > 0, den, 1.0)
    if trace is not None:
        trace["decoded_kv_bytes"] = int(np.asarray(k_hat).nbytes + np.asarray(v_hat).nbytes)
        trace["score_bytes"] = int(scores.nbytes)
    return out.reshape(q.shape)


def merge_blocks(score_blocks, value_blocks, rescale_z=True, rescale_u=True):
    """Online softmax over a sequence of blocks, carrying ``(m, z, u)``.

    ``score_blocks[i]`` is ``[..., L_i]`` (float64 scores of one block),
    ``value_blocks[i]`` is ``[L_i, D]`` or ``[..., L_i, D]``.  Returns the
    final ``u / z`` and the list of ``(m, z, u)`` states after each block.

    [BKD] "Do not average independently normalized blocks" and [RL] "why
    FlashAttention need not keep the whole heat map":
        m_new = max(m_old, max(block scores))
        a     = exp(m_old - m_new)
        z_new = a*z_old + sum(exp(block scores - m_new))
        u_new = a*u_old + exp(block scores - m_new) @ block V
        output = u / z
    starting from m = -inf, z = u = 0.  Empty blocks are skipped, so
    -inf - (-inf) is never formed ([RL] same section).  Masked scores are
    -inf: they add nothing to the max or the sums, and a row that has seen
    no legal key yet stays at (-inf, 0, 0) and ends as zeros.  ``rescale_z`` and
    ``rescale_u`` exist only for the ablation the pages ask for ([BKD] "Use
    the failure to choose the next question", [TOS] "exercises"): dropping
    either rescale must break the result.
    """
    m = z = u = None
    states = []
    for s_blk, v_blk in zip(score_blocks, value_blocks):
        s_blk = np.asarray(s_blk, dtype=np.float64)
        v_blk = np.asarray(v_blk, dtype=np.float64)
        if s_blk.shape[-1] == 0:
            continue
        blk_max = s_blk.max(axis=-1)
        if m is None:
            m_new = blk_max
            z = np.zeros_like(blk_max)
            u = np.zeros(s_blk.shape[:-1] + (v_blk.shape[-1],), dtype=np.float64)
            a = np.zeros_like(blk_max)
        else:
            m_new = np.maximum(m, blk_max)
            a = np.exp(m - np.where(np.isfinite(m_new), m_new, 0.0))
        ref = np.where(np.isfinite(m_new), m_new, 0.0)   # rows with no legal key yet
        p = np.exp(s_blk - ref[..., None])
        z = (a * z if rescale_z else z) + p.sum(axis=-1)
        u = (a[..., None] * u if rescale_u else u) + np.matmul(p[..., None, :], v_blk)[..., 0, :]
        m = m_new
        states.append((m.copy(), z.copy(), u.copy()))
    if m is None:
        raise ValueError("no non-empty block: a row with no key is undefined")
    return u / np.where(z > 0, z, 1.0)[..., None], states


def attend_blocked(q, k_hat, v_hat, block, sm_scale=None, rescale_z=True,
                   rescale_u=True, trace=None, causal=False):
    """Blocked attention: score ``block`` tokens at a time and merge them with
    :func:`merge_blocks`.  Same inputs and output as :func:`attend_dense`.

    [BKD] "Do not average independently normalized blocks" (32-token blocks)
    and [TOS] "exercises" (a block length such as 7 that does not divide N:
    the last block is shorter).  Decoding is elementwise, so slicing a block
    of an already decoded cache gives the same values as decoding that block
    from its codes.  ``causal``: scores outside ``causal_mask`` are -inf.
    """
    d = q.shape[-1]
    scale = default_scale(d) if sm_scale is None else float(sm_scale)
    k64 = np.asarray(k_hat, dtype=np.float64)
    v64 = np.asarray(v_hat, dtype=np.float64)
    rows = _gqa_rows(np.asarray(q, dtype=np.float64), k64.shape[1])
    n = k64.shape[-2]
    visible = np.tile(causal_mask(n, q.shape[2]), (rows.shape[2] // q.shape[2], 1))
    score_blocks, value_blocks = [], []
    for start in range(0, n, block):
        k_blk = k64[..., start:start + block, :]
        s_blk = np.matmul(rows, np.swapaxes(k_blk, -1, -2)) * scale
        if causal:
            s_blk = np.where(visible[:, start:start + block], s_blk, -np.inf)
        score_blocks.append(s_blk)
        value_blocks.append(v64[..., None, start:start + block, :])
        if trace is not None and start == 0:
            kb = np.asarray(k_hat)[..., start:start + block, :]
            vb = np.asarray(v_hat)[..., start:start + block, :]
            trace["decoded_kv_bytes"] = int(kb.nbytes + vb.nbytes)
            trace["score_bytes"] = int(score_blocks[0].nbytes)
    # value blocks are [B, Hkv, 1, L, D]; matmul broadcasts them over rows.
    out, _ = merge_blocks(score_blocks, value_blocks, rescale_z, rescale_u)
    return out.reshape(q.shape)


def block_average(score_blocks, value_blocks):
    """The wrong baseline: softmax each block on its own, then average the
    block outputs with equal weight.

    [BKD] "Do not average independently normalized blocks" and [TOS] "why
    normalizing each block and averaging is wrong": this forces every block's
    mass to 1 and loses the relative scores between blocks.  Kept only for
    the negative test.
    """
    outs = []
    for s_blk, v_blk in zip(score_blocks, value_blocks):
        s_blk = np.asarray(s_blk, dtype=np.float64)
        w = np.exp(s_blk - s_blk.max(axis=-1, keepdims=True))
        outs.append(np.matmul(w / w.sum(axis=-1, keepdims=True), np.asarray(v_blk, np.float64)))
    return sum(outs) / len(outs)


def split_bounds(n: int, num_splits: int):
    """Token ranges of a split-KV pass: ``num_splits`` contiguous chunks of
    ``ceil(n / num_splits)`` tokens (trailing chunks may be short or empty)."""
    chunk = -(-n // num_splits)
    return [(min(s * chunk, n), min((s + 1) * chunk, n)) for s in range(num_splits)]


def attend_split(q, k_hat, v_hat, num_splits, sm_scale=None):
    """Split-KV attention: each token chunk yields its own ``(m, z, u)`` per
    row, and the chunks are combined with the same rescale.

    [RL] "two stops of the online accumulation": partial statistics z and u
    are composable once brought to a common exponent base;
        M = max_s m_s,  Z = sum_s exp(m_s - M) z_s,  U = sum_s exp(m_s - M) u_s,
        out = U / Z.
    Empty chunks carry m = -inf and are skipped ([RL] "why FlashAttention
    need not keep the whole heat map").
    """
    d = q.shape[-1]
    scale = default_scale(d) if sm_scale is None else float(sm_scale)
    k64 = np.asarray(k_hat, dtype=np.float64)
    v64 = np.asarray(v_hat, dtype=np.float64)
    rows = _gqa_rows(np.asarray(q, dtype=np.float64), k64.shape[1])
    parts = []
    for lo, hi in split_bounds(k64.shape[-2], num_splits):
        if hi <= lo:
            continue
        s = np.matmul(rows, np.swapaxes(k64[..., lo:hi, :], -1, -2)) * scale
        m = s.max(axis=-1)
        p = np.exp(s - m[..., None])
        parts.append((m, p.sum(axis=-1), np.matmul(p, v64[..., lo:hi, :])))
    big_m = np.max(np.stack([m for m, _, _ in parts]), axis=0)
    big_z = sum(np.exp(m - big_m) * z for m, z, _ in parts)
    big_u = sum(np.exp(m - big_m)[..., None] * u for m, _, u in parts)
    return (big_u / big_z[..., None]).reshape(q.shape)


def attend_packed(q, k_codes, k_scales, v_codes, v_scales, n, bits, group, sm_scale=None,
                  causal=False):
    """The oracle of the fused path: decode the whole packed cache to float32
    ([KPG] "what a byte holds"), promote to float64 and run dense attention
    ([BKD] "Compare equivalent representations first")."""
    b, hkv = k_codes.shape[0], k_codes.shape[1]
    d = q.shape[-1]
    shape = (b, hkv, n, d)
    k_hat = dequant_k(k_codes, k_scales, shape, bits, group)
    v_hat = dequant_v(v_codes, v_scales, shape, bits, group)
    return attend_dense(q, k_hat, v_hat, sm_scale, causal=causal)


def attend_window(q, k, v, window, bits, group, sm_scale=None, causal=False):
    """Attention over a mixed cache: the oldest ``N - window`` tokens packed,
    the most recent ``window`` tokens kept in float32.

    [KPG] "exercises and common mistakes" announces the study of leaving
    limited high-precision room to the most recent tokens, keeping the same
    packed format, and "accuracy and space on the same input" builds the
    early / late biased inputs for it.  Reading: the packed part is the
    packed tensor of the first ``N - window`` tokens on their own (its last
    short group zero-padded, as for any length), the window tokens enter
    attention unquantized, and attention runs over all N tokens in float64
    ([BKD] "Compare equivalent representations first").
    Parity: pinned in tests/test_oracle_window.py (window 0 is the packed
    path, window N the float32 path, and the decoded cache is the packed
    prefix followed by the raw window).
    """
    n, d = k.shape[-2], k.shape[-1]
    npk = n - window
    k_hat = np.array(k, dtype=np.float32)
    v_hat = np.array(v, dtype=np.float32)
    if npk > 0:
        shape = k.shape[:-2] + (npk, d)
        k_hat[..., :npk, :] = dequant_k(*pack_k(k[..., :npk, :], bits, group), shape, bits, group)
        v_hat[..., :npk, :] = dequant_v(*pack_v(v[..., :npk, :], bits, group), shape, bits, group)
    return attend_dense(q, k_hat, v_hat, sm_scale, causal=causal)


# ---------------------------------------------------------------------------
# Byte ledgers and error measures
# ---------------------------------------------------------------------------

def packed_payload_bytes(n: int, d: int, bits: int, group: int, shape_record=True) -> int:
    """Bytes of one head's packed K and V: code bytes + float32 scales (+ the
    two int32[2] shape records).

    [KPG] "what a byte holds" (float32 scales and an int32 two-dim shape are
    kept and counted) and the payload table of "accuracy and space on the same
    input".
    """
    npad = -(-n // group) * group
    dpad = -(-d // group) * group
    code_bytes = (d * npad + n * dpad) * bits // 8
    scale_bytes = 4 * (d * npad // group + n * dpad // group)
    return code_bytes + scale_bytes + (2 * 2 * 4 if shape_record else 0)


def kv_bytes(layers: int, batch: int, n: int, hkv: int, dh: int, s: float) -> float:
    """[RL] "KV payload units must be written in full":
    KV bytes = 2 * L * B * n * H_kv * d_h * s, with s bytes per element."""
    return 2 * layers * batch * n * hkv * dh * s


def bytes_per_element(bits: int, group: int) -> float:
    """Per-element storage of the packed cache in the formula above: the code
    plus its share of one float32 scale, ``bits/8 + 4/group``."""
    return bits / 8 + 4 / group


def rel_l2(approx, ref) -> float:
    """Output relative L2 error of one input: ||approx - ref||_F / ||ref||_F
    ([KPG] "accuracy and space on the same input": computed per input, then
    averaged over inputs)."""
    a = np.asarray(approx, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(a - r) / np.linalg.norm(r))
