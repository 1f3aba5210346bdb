"""Token-group storage of the value side at d = 128 (oracle side, CPU only).

The value codes of four neighbouring slots, and the value sign bits of eight,
share bytes so that the decode scan reads ready-made table indices.  These
tests pin the oracle's definition of that format: every bit of every slot's
record has its own place inside its group (a bijection), and storing records
that way changes nothing that is computed from them.
"""
import ctypes as C

import numpy as np
import pytest

from oracle import ref


def _code_bit(bits, slot, c, i):
    by, bt = C.c_size_t(), C.c_int()
    ref.lib().orc_vgroup_code_bit(bits, slot, c, i, C.byref(by), C.byref(bt))
    return by.value, bt.value


def _sign_bit(slot, k):
    by, bt = C.c_size_t(), C.c_int()
    ref.lib().orc_vgroup_sign_bit(slot, k, C.byref(by), C.byref(bt))
    return by.value, bt.value


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_code_positions_fill_each_quad_exactly_once(bits):
    rec = 16 * bits
    q = 5                                    # any quad: positions are relative to 4 q rec
    seen = set()
    for r in range(4):
        for c in range(128):
            for i in range(bits):
                by, bt = _code_bit(bits, 4 * q + r, c, i)
                assert 4 * q * rec <= by < 4 * (q + 1) * rec and 0 <= bt < 8
                seen.add((by, bt))
    assert len(seen) == 4 * rec * 8


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_pieces_hold_eight_coordinates_of_the_quad(bits):
    """Piece n (bytes 4 b n .. 4 b n + 4 b - 1 of the quad) holds exactly the
    codes of coordinates 8 n .. 8 n + 7 of the quad's four slots."""
    pb = 4 * bits
    for c in range(128):
        for r in range(4):
            for i in range(bits):
                by, _ = _code_bit(bits, r, c, i)
                assert by // pb == c // 8


def test_sign_positions_fill_each_octet_exactly_once():
    o = 3
    seen = set()
    for e in range(8):
        for k in range(128):
            by, bt = _sign_bit(8 * o + e, k)
            assert 128 * o <= by < 128 * (o + 1)
            assert bt == e and by - 128 * o == k
            seen.add((by, bt))
    assert len(seen) == 128 * 8


def test_pair_fields_of_three_bit_codes():
    """Width 3: the codes of slots 2p and 2p + 1 of a quad form one 6-bit pair
    field per coordinate; fields 0..11 of a piece are the high 6 bits of its
    bytes and fields 12..15 are spread over bits 0 and 1 of three bytes."""
    for c in range(8):                        # piece 0, j = c
        for p in range(2):
            u = 2 * c + p
            pos = [_code_bit(3, 2 * p + q, c, i) for q in range(2) for i in range(3)]
            if u < 12:
                assert pos == [(u, 2 + b) for b in range(6)]
            else:
                m = u - 12
                assert pos == [(m, 0), (m, 1), (4 + m, 0), (4 + m, 1), (8 + m, 0), (8 + m, 1)]


def _caches(scheme, n, values, cap=48):
    ks, vs = ref.scheme_sides(scheme, n)
    return (ref.OracleCache(1, 2, cap, 128, ks, 128),
            ref.OracleCache(1, 2, cap, 128, vs, 128, values=values))


@pytest.mark.parametrize("scheme,n", [("KQV", 4), ("KQV", 3), ("KQV", 2), ("KV", 4), ("KV", 1),
                                      ("QKQV", 4)])
def test_grouped_storage_changes_no_result(scheme, n):
    """Two writes that start and end inside groups, into a per-slot and a
    grouped value side: every slot's record reads back the same, the
    reconstructions and the attention outputs are equal, and the second write
    leaves the first one's slots alone."""
    rng = np.random.default_rng(11)
    S = rng.standard_normal((128, 128)).astype(np.float32)
    Sb = np.array([ref.f32_to_bf16_bits(float(x)) for x in S.ravel()], np.uint16).reshape(128, 128)
    x1 = rng.standard_normal((1, 2, 7, 128)).astype(np.float32)
    x2 = rng.standard_normal((1, 2, 22, 128)).astype(np.float32)
    (k0, v0), (k1, v1) = _caches(scheme, n, False), _caches(scheme, n, True)
    assert v1.grouped == 1 and v0.grouped == 0
    for kc, vc in ((k0, v0), (k1, v1)):
        for cache in (kc, vc):
            cache.quantize(x1, 5, Sb)
            cache.quantize(x2, 12, Sb)
    side = v1.side
    rb, sb = 128 * side.bits // 8, 16
    rec = np.zeros(rb, np.uint8)
    sg = np.zeros(sb, np.uint8)
    for u in range(2):
        for slot in range(5, 34):
            gs = u * 48 + slot
            ref.lib().orc_load_record(ref._p(v1.codes), ref._p(v1.signs), 1, gs, 128, side.bits,
                                      side.qjl, 128, ref._p(rec), ref._p(sg))
            assert np.array_equal(rec, v0.codes[0, u, slot])
            if side.qjl:
                assert np.array_equal(sg, v0.signs[0, u, slot])
    assert np.array_equal(v1.norm, v0.norm)
    np.testing.assert_array_equal(v1.dequantize(5, 29, Sb), v0.dequantize(5, 29, Sb))
    q = rng.standard_normal((1, 4, 128)).astype(np.float32)
    a0 = ref.attention(k0, v0, q, 34, Sb)
    a1 = ref.attention(k1, v1, q, 34, Sb)
    np.testing.assert_array_equal(a0, a1)


def test_grouped_value_side_needs_whole_blocks():
    ks, vs = ref.scheme_sides("KQV", 4)
    with pytest.raises(ValueError):
        ref.OracleCache(1, 1, 40, 128, vs, 128, values=True)
    assert ref.OracleCache(1, 1, 40, 64, vs, 64, values=True).grouped == 0
