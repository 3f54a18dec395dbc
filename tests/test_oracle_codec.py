"""Pins of the oracle's quantizer, packer and decoder against facts the pages
fix, closed forms, invariants and an independent brute force.  CPU only."""
import struct

import numpy as np
import pytest

from oracle import kvq_oracle as O
from workloads import WORKLOADS, make_crafted, make_qkv


def f32(x: float) -> float:
    """Round a Python float to the nearest IEEE float32 (an independent route
    to float32 arithmetic: a float64 quotient rounded once to float32 is the
    correctly rounded float32 quotient, since 53 >= 2*24 + 2)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def brute_quantize_group(vals, bits):
    """Scalar re-derivation of one group's quantization: scale = max|x|/qmax
    (1 when that is 0), then for every element the code c in [-qmax, qmax]
    nearest to x/scale, ties to the even code."""
    qmax = O.QMAX[bits]
    m = max(abs(f32(v)) for v in vals)
    s = f32(m / qmax)
    if s == 0.0:
        s = 1.0
    codes = []
    for v in vals:
        t = f32(f32(v) / s)
        best = None
        for c in range(-qmax, qmax + 1):
            key = (abs(t - c), c % 2)  # nearest, then even
            if best is None or key < best[0]:
                best = (key, c)
        codes.append(best[1] + qmax)
    return codes, s


# --- worked example of the page --------------------------------------------

def test_nibble_pack_d2(golden):
    g = golden("nibble_pack_d2.json")
    packed = O.pack_nibbles(np.array([g["stored_low"], g["stored_high"]], dtype=np.uint8))
    assert packed.tolist() == [int(g["byte_hex"], 16)]
    lo, hi = O.unpack_nibbles(packed).tolist()
    assert (lo, hi) == (g["stored_low"], g["stored_high"])
    assert (lo - g["offset"], hi - g["offset"]) == (g["code_low"], g["code_high"])
    # &15 and >>4 by hand
    b = int(g["byte_hex"], 16)
    assert (b & 15, b >> 4) == (2, 13)


def test_decode_of_d2_with_unit_scale(golden):
    g = golden("nibble_pack_d2.json")
    codes = np.array([[int(g["byte_hex"], 16)]], dtype=np.uint8)   # one row, two elements
    scales = np.array([[1.0]], dtype=np.float32)
    x = O.dequant(codes, scales, (1, 2), -1, 4, 2)
    assert x.tolist() == [[g["code_low"], g["code_high"]]]


# --- special cases ------------------------------------------------------------

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [8, 32])
@pytest.mark.parametrize("axis", [-2, -1])
def test_all_zero_decodes_to_zero(bits, group, axis):
    x = make_crafted("zeros")
    with np.errstate(all="raise"):
        codes, scales = O.pack(x, axis, bits, group)
        xd = O.dequant(codes, scales, x.shape, axis, bits, group)
    assert np.all(scales == 1.0)
    assert np.all(xd == 0.0) and not np.any(np.signbit(xd))
    assert np.all(O.unpack_stored(codes, x.shape, axis, bits, group) == O.QMAX[bits])


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [8, 32])
@pytest.mark.parametrize("axis", [-2, -1])
def test_ragged_35x13_round_trip(bits, group, axis):
    x = make_crafted("ragged")
    codes, scales = O.pack(x, axis, bits, group)
    length = x.shape[axis]
    other = x.shape[1] if axis == -2 else x.shape[0]
    padded = -(-length // group) * group
    assert codes.shape == (other, padded * bits // 8)
    assert scales.shape == (other, padded // group)
    xd = O.dequant(codes, scales, x.shape, axis, bits, group)
    assert xd.shape == (35, 13)
    stored = O.unpack_stored(codes, x.shape, axis, bits, group)
    assert stored.shape == (35, 13)
    # padding positions hold the zero code
    if bits == 4:
        full = O.unpack_nibbles(codes).reshape(other, padded)
    else:
        full = codes.reshape(other, padded)
    assert np.all(full[:, length:] == O.QMAX[bits])
    # elementwise error bound of round-to-nearest
    s_el = O.expand_scales(scales, x.shape, axis, group)
    assert np.all(np.abs(x.astype(np.float64) - xd) <= s_el.astype(np.float64) * (0.5 + 1e-6))


def test_subnormal_groups_and_scale_underflow():
    x = make_crafted("tiny")
    codes, scales = O.pack(x, -1, 4, 32)
    # row 1's max|x|/7 underflows to zero: scale falls back to 1, codes all zero
    assert scales[1, 0] == 1.0
    assert np.all(O.unpack_stored(codes, x.shape, -1, 4, 32)[1] == 7)
    # row 0 keeps a subnormal scale and still reaches +-7
    assert 0 < scales[0, 0] < np.finfo(np.float32).tiny
    st = O.unpack_stored(codes, x.shape, -1, 4, 32)[0]
    assert st.min() == 0 or st.max() == 14


# --- invariants and closed forms ------------------------------------------------

@pytest.mark.parametrize("bits,group", [(4, 8), (4, 32), (8, 8), (8, 32)])
def test_code_range_and_extremes(bits, group):
    q, k, v = make_qkv(WORKLOADS["single_n512"], 0)
    for x, axis in ((k[0, 0], -2), (v[0, 0], -1)):
        codes, scales = O.pack(x, axis, bits, group)
        grouped = O.group_last(O.unpack_stored(codes, x.shape, axis, bits, group), axis, group)
        qmax = O.QMAX[bits]
        assert grouped.max() <= 2 * qmax  # 15 (255) never appears
        # every group holds its max at +-qmax
        hits = (grouped == 0) | (grouped == 2 * qmax)
        assert np.all(hits.any(axis=-1))


def test_really_packed_half_of_8bit():
    x = make_qkv(WORKLOADS["single_n128"], 1)[1][0, 0]
    c4, _ = O.pack_k(x, 4, 32)
    c8, _ = O.pack_k(x, 8, 32)
    assert c4.nbytes * 2 == c8.nbytes


@pytest.mark.parametrize("bits", [4, 8])
def test_sign_symmetry(bits):
    x = make_qkv(WORKLOADS["single_n128"], 2)[2][0, 0]
    c1, s1 = O.pack_v(x, bits, 8)
    c2, s2 = O.pack_v(-x, bits, 8)
    st1 = O.unpack_stored(c1, x.shape, -1, bits, 8).astype(int)
    st2 = O.unpack_stored(c2, x.shape, -1, bits, 8).astype(int)
    assert np.array_equal(s1, s2)
    assert np.array_equal(st2, 2 * O.QMAX[bits] - st1)


@pytest.mark.parametrize("shift", [-3, 5])
def test_power_of_two_scaling(shift):
    x = make_qkv(WORKLOADS["single_n128"], 0)[1][0, 0]
    c1, s1 = O.pack_k(x, 4, 32)
    c2, s2 = O.pack_k(np.ldexp(x, shift).astype(np.float32), 4, 32)
    assert np.array_equal(c1, c2)
    assert np.array_equal(np.ldexp(s1, shift), s2)


def test_ties_round_half_even():
    x = make_crafted("ties")
    codes, scales = O.pack(x, -1, 4, 32)
    assert scales[0, 0] == 1.0  # max|x| = 7
    st = O.unpack_stored(codes, x.shape, -1, 4, 32).astype(int) - 7
    # first five entries of the crafted row: 7, 0.5, 1.5, 2.5, -2.5
    assert st[0, :5].tolist() == [7, 0, 2, 2, -2]
    assert st[1, :5].tolist() == [-7, 0, -2, -2, 2]


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("group", [8, 32])
def test_brute_force_quantizer(bits, group):
    rng = np.random.default_rng(123)
    x = rng.standard_normal((6, 2 * group + 6), dtype=np.float32)
    x[0, 3] = 0.0
    x[2] *= np.float32(1e3)
    codes, scales = O.pack(x, -1, bits, group)
    stored = O.unpack_stored(codes, x.shape, -1, bits, group)
    for r in range(x.shape[0]):
        row = x[r].tolist()
        row += [0.0] * ((-len(row)) % group)
        for gi in range(len(row) // group):
            vals = row[gi * group:(gi + 1) * group]
            want_codes, want_s = brute_quantize_group(vals, bits)
            assert scales[r, gi] == np.float32(want_s)
            got = [int(c) for c in stored[r, gi * group:(gi + 1) * group]] if (gi + 1) * group <= x.shape[1] \
                else [int(c) for c in stored[r, gi * group:]]
            assert got == want_codes[:len(got)]


def test_brute_force_dequant_matches_float32_multiply():
    x = make_qkv(WORKLOADS["single_n128"], 0)[1][0, 0]
    codes, scales = O.pack_k(x, 4, 32)
    xd = O.dequant_k(codes, scales, x.shape, 4, 32)
    st = O.unpack_stored(codes, x.shape, -2, 4, 32)
    for n in range(0, 128, 37):
        for d in range(0, 32, 5):
            want = f32((int(st[n, d]) - 7) * float(scales[d, n // 32]))
            assert float(xd[n, d]) == want


def test_k_layout_is_channel_major():
    """K codes: byte i of channel d's row holds tokens 2i (low) and 2i+1
    (high): groups run along tokens inside a channel."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 4), dtype=np.float32)
    codes, scales = O.pack_k(x, 4, 32)
    assert codes.shape == (4, 32) and scales.shape == (4, 2)
    for d in range(4):
        for t in range(64):
            want, s = brute_quantize_group(x[(t // 32) * 32:(t // 32 + 1) * 32, d].tolist(), 4)
            byte = int(codes[d, t // 2])
            nib = byte & 15 if t % 2 == 0 else byte >> 4
            assert nib == want[t % 32]


def test_v_layout_is_token_major():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 16), dtype=np.float32)
    codes, scales = O.pack_v(x, 4, 8)
    assert codes.shape == (3, 8) and scales.shape == (3, 2)
    for n in range(3):
        for f in range(16):
            want, _ = brute_quantize_group(x[n, (f // 8) * 8:(f // 8 + 1) * 8].tolist(), 4)
            byte = int(codes[n, f // 2])
            assert (byte & 15 if f % 2 == 0 else byte >> 4) == want[f % 8]


# --- byte ledgers -----------------------------------------------------------------

def test_byte_ledger(golden):
    g = golden("byte_ledger.json")
    n, d = g["n"], g["d"]
    for key, want in g["payload_bytes"].items():
        bits, group = map(int, key.split("_"))
        assert O.packed_payload_bytes(n, d, bits, group) == want
        # and the arrays the packer really produces add up to it
        k = np.zeros((n, d), np.float32)
        kc, ks = O.pack_k(k, bits, group)
        vc, vs = O.pack_v(k, bits, group)
        assert kc.nbytes + ks.nbytes + vc.nbytes + vs.nbytes + 16 == want
    assert 2 * n * d * 4 == g["float32_kv_bytes"]
    assert O.packed_payload_bytes(n, d, 4, 32, shape_record=False) - 4 * (d * n // 32 + n * d // 32) \
        == g["codes_only_4bit_g32"]
    red = 100 * (1 - g["payload_bytes"]["4_32"] / g["float32_kv_bytes"])
    assert round(red, 1) == g["reduction_4bit_g32_percent"]
    assert round(red, 1) != g["not_reduction_percent"]


def test_kv_bytes_formula(golden):
    g = golden("kv_bytes_example.json")
    b = O.kv_bytes(g["L"], g["B"], g["n"], g["H_kv"], g["d_h"], g["s"])
    assert b == g["kv_bytes"] == g["mib"] * 2 ** 20
    mha = O.kv_bytes(g["L"], g["B"], g["n"], g["mha_H_kv"], g["d_h"], g["s"])
    assert mha == g["mha_gib"] * 2 ** 30
    # the packed format's per-element bytes reproduce the packer's array sizes
    w = WORKLOADS["gqa_n4096"]
    per_layer = O.kv_bytes(1, w.B, w.N, w.Hkv, w.D, O.bytes_per_element(4, 32))
    assert per_layer == w.B * w.Hkv * (O.packed_payload_bytes(w.N, w.D, 4, 32, shape_record=False))
    assert per_layer == 41943040


# --- block byte order of the device layout ------------------------------------
# The pages leave the byte order open; the library's block order is checked
# here against the canonical arrays directly (no reshape shared with
# store_k / store_v): first in the form the matrix-core kernel consumes it,
# then element by element through the byte formula written in include/kvq.h.

def _random_cache(n, d, seed=11):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((1, 1, n, d), dtype=np.float32),
            rng.standard_normal((1, 1, n, d), dtype=np.float32))


def test_store_k_gives_matrix_core_rows():
    """4-bit, D=128: the 8 bytes at k-step ks*512 + lane*8 of a block are the
    bytes of token pair 16*blk + n (n = lane % 16) for channels
    ks*32 + 8*(lane // 16) + e, e = 0..7."""
    n_tok, d = 96, 128
    k, _ = _random_cache(n_tok, d)
    kc, ks = O.pack_k(k, 4, 32)
    st, sst = O.store_k(kc, ks, n_tok, d, 4, 32)
    assert st.shape == (1, 1, 3, 2048)
    for blk in range(3):
        for ks_ in range(4):
            for lane in range(64):
                n, q = lane % 16, lane // 16
                got = st[0, 0, blk, ks_ * 512 + lane * 8: ks_ * 512 + lane * 8 + 8]
                want = [kc[0, 0, ks_ * 32 + 8 * q + e, 16 * blk + n] for e in range(8)]
                assert list(got) == want
    assert np.array_equal(sst[0, 0].T, ks[0, 0])      # group-major scales


def test_store_v_gives_matrix_core_columns():
    """4-bit, D=128: the 8 bytes at q*512 + g*128 + n*8 of a block are byte
    column 16g + n of tokens 32*blk + 8q + e, e = 0..7; the V scales of
    value group G for tokens 8q..8q+7 sit at G*32 + 8q .. + 7."""
    n_tok, d = 64, 128
    _, v = _random_cache(n_tok, d)
    vc, vs = O.pack_v(v, 4, 32)
    st, sst = O.store_v(vc, vs, n_tok, d, 4, 32)
    assert st.shape == (1, 1, 2, 2048) and sst.shape == (1, 1, 2, 128)
    for blk in range(2):
        for q in range(4):
            for g in range(4):
                for n in range(16):
                    off = q * 512 + g * 128 + n * 8
                    want = [vc[0, 0, 32 * blk + 8 * q + e, 16 * g + n] for e in range(8)]
                    assert list(st[0, 0, blk, off:off + 8]) == want
            for G in range(4):
                assert np.array_equal(sst[0, 0, blk, G * 32 + 8 * q: G * 32 + 8 * q + 8],
                                      vs[0, 0, 32 * blk + 8 * q: 32 * blk + 8 * q + 8, G])


def _nibble(byte, hi, bits):
    return (byte >> 4 if hi else byte & 15) if bits == 4 else byte


@pytest.mark.parametrize("bits,group", [(4, 8), (4, 32), (8, 8), (8, 6), (4, 2), (4, 64)])
@pytest.mark.parametrize("n,d", [(35, 13), (1, 1), (64, 32), (33, 40)])
def test_store_matches_header_formula(bits, group, n, d):
    """Every element through the byte formula of include/kvq.h, every other
    position holds the zero code, padded V scales are 1."""
    k, v = _random_cache(n, d, seed=n * 100 + d)
    kc, ks = O.pack_k(k, bits, group)
    vc, vs = O.pack_v(v, bits, group)
    sk, sks = O.store_k(kc, ks, n, d, bits, group)
    sv, svs = O.store_v(vc, vs, n, d, bits, group)
    kst = O.unpack_stored(kc, k.shape, -2, bits, group)[0, 0]
    vst = O.unpack_stored(vc, v.shape, -1, bits, group)[0, 0]
    nb, d8, dpad = -(-n // 32), -(-d // 8), -(-d // group) * group
    kcols, vcols = 32 * bits // 8, dpad * bits // 8
    kflat, vflat = sk[0, 0].reshape(-1), sv[0, 0].reshape(-1)
    kseen, vseen = set(), set()
    for t in range(n):
        for c in range(d):
            j = (t % 32) // 2 if bits == 4 else t % 32
            kb = (t // 32) * d8 * kcols * 8 + ((c // 8) * kcols + j) * 8 + c % 8
            assert _nibble(int(kflat[kb]), t % 2, bits) == kst[t, c]
            kseen.add((kb, t % 2 if bits == 4 else 0))
            col = c // 2 if bits == 4 else c
            vb = (t // 32) * 4 * vcols * 8 + (((t % 32) // 8) * vcols + col) * 8 + t % 8
            assert _nibble(int(vflat[vb]), c % 2, bits) == vst[t, c]
            vseen.add((vb, c % 2 if bits == 4 else 0))
            assert sks[0, 0, t // group, c] == ks[0, 0, c, t // group]
            vsi = ((t // 32) * (dpad // group) + c // group) * 32 + t % 32
            assert svs[0, 0].reshape(-1)[vsi] == vs[0, 0, t, c // group]
    zero = O.QMAX[bits]
    halves = (0, 1) if bits == 4 else (0,)
    for flat, seen in ((kflat, kseen), (vflat, vseen)):
        for b in range(flat.size):
            for h in halves:
                if (b, h) not in seen:
                    assert _nibble(int(flat[b]), h, bits) == zero
    vsflat = svs[0, 0].reshape(nb, dpad // group, 32)
    assert np.all(vsflat[:, :, :][np.arange(nb * 32).reshape(nb, 1, 32).repeat(dpad // group, 1) >= n] == 1.0)
