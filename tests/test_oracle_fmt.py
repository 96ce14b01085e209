"""Pins of the packed layout (oracle/fmt.py).

The layout is this project's own definition, so what can be pinned is that
it is a lossless, padding-free bijection, that b = 2 and b = 4 coincide with
plain LSB-first packing built independently here with byte arithmetic, and a
few units worked out by hand from the layout's definition."""
import numpy as np
import pytest

from oracle import fmt


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6])
def test_unit_positions_are_a_bijection(b):
    pos = fmt.unit_positions(b)
    assert pos.shape == (32, b, 2)
    flat = pos[:, :, 0] * 32 + pos[:, :, 1]
    assert np.all((pos[:, :, 0] >= 0) & (pos[:, :, 0] < b))
    assert np.all((pos[:, :, 1] >= 0) & (pos[:, :, 1] < 32))
    assert len(np.unique(flat)) == 32 * b          # every bit of the unit used once


@pytest.mark.parametrize("b", [2, 3, 4, 5, 6])
def test_pack_roundtrip_and_size(b):
    rng = np.random.default_rng(b)
    q = rng.integers(0, 1 << b, size=(7, 32 * 9), dtype=np.uint8)
    words = fmt.pack_codes(q, b)
    assert words.shape == (7, 9 * b) and words.dtype == np.uint32
    assert words.nbytes == fmt.codes_bytes(7, 32 * 9, b)
    assert np.array_equal(fmt.unpack_codes(words, 7, 32 * 9, b), q)
    with pytest.raises(ValueError):
        fmt.pack_codes(np.full((1, 32), 1 << b, dtype=np.uint8), b)


def test_b4_b2_are_plain_lsb_first():
    rng = np.random.default_rng(0)
    q = rng.integers(0, 16, size=(3, 64), dtype=np.uint8)
    plain4 = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)        # two nibbles per byte
    assert np.array_equal(fmt.pack_codes(q, 4).view(np.uint8), plain4)
    q = rng.integers(0, 4, size=(3, 64), dtype=np.uint8)
    plain2 = (q[:, 0::4] | (q[:, 1::4] << 2) | (q[:, 2::4] << 4) | (q[:, 3::4] << 6)).astype(np.uint8)
    assert np.array_equal(fmt.pack_codes(q, 2).view(np.uint8), plain2)


def unit_with(b, code_index, value):
    q = np.zeros((1, 32), dtype=np.uint8)
    q[0, code_index] = value
    return list(int(w) for w in fmt.pack_codes(q, b)[0])


def test_hand_worked_units():
    # b=3, code 30 = 0b101: spare bit 15 of words 0 and 2 (bit 1 is 0).
    assert unit_with(3, 30, 0b101) == [0x8000, 0, 0x8000]
    # b=3, code 31 = 0b011: bit 31 of words 0 and 1.
    assert unit_with(3, 31, 0b011) == [0x80000000, 0x80000000, 0]
    # b=3, code 7: word 0, high half (7 % 10 = 7 >= 5), field 2 -> bits 16+6.
    assert unit_with(3, 7, 0b111) == [0b111 << 22, 0, 0]
    # b=5, code 7 = 22: word 1, low half, field 1 -> bits 5..9 of word 1.
    assert unit_with(5, 7, 22) == [0, 22 << 5, 0, 0, 0]
    # b=5, code 31 = 0b10001: bit 31 of word 0 and word 4.
    assert unit_with(5, 31, 0b10001) == [0x80000000, 0, 0, 0, 0x80000000]
    # b=6, code 29 = 0b110001: p = 1, high half; low bits -> word 1 bit 28,
    # top two bits -> word 4 bits 30, 31.
    assert unit_with(6, 29, 0b110001) == [0, 1 << 28, 0, 0, 0xC0000000, 0]
    # b=6, code 5 = 63: word 1 (5 // 4), low half, field 1 -> bits 6..11.
    assert unit_with(6, 5, 63) == [0, 63 << 6, 0, 0, 0, 0]
    # b=6, code 26 = 0b100000: p = 2, low half; bit 5 -> word 5, bit 12+1.
    assert unit_with(6, 26, 0b100000) == [0, 0, 0, 0, 0, 1 << 13]


def test_meta_roundtrip():
    s = np.array([[0.5, 0.001]], dtype=np.float16)
    o = np.array([[-0.25, 3.0]], dtype=np.float16)
    m = fmt.pack_meta(s, o)
    assert m[0, 0] == (0x3800 | (0xB400 << 16))
    s2, o2 = fmt.unpack_meta(m)
    assert np.array_equal(s2, s) and np.array_equal(o2, o)
