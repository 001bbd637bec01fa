"""Pins of the record layout (reading R18 of the ambiguity register: the
pages fix no byte order, so the record's layout is a stated convention):

* 4-bit codes: element 2j in the low nibble of byte j, element 2j + 1 in
  the high nibble;
* bit-planes and masks: bit k of byte j belongs to element 8j + k.

The packing helpers are checked against bytes written out by hand and
against a per-element loop over the convention, so that a swap of the
nibble or bit order in both the packing and the unpacking helper (which a
round trip would not see) fails here."""
import numpy as np

import oracle


def test_pack_nibbles_hand_written_bytes():
    assert oracle.pack_nibbles([0x1, 0x2, 0x3, 0xF]).tolist() == [0x21, 0xF3]
    assert oracle.pack_nibbles([0xA, 0x0, 0x0, 0xB, 0x8, 0x7]).tolist() == [0x0A, 0xB0, 0x78]


def test_unpack_nibbles_hand_written_bytes():
    assert oracle.unpack_nibbles(np.array([0x21, 0xF3], dtype=np.uint8), 4).tolist() == [0x1, 0x2, 0x3, 0xF]
    assert oracle.unpack_nibbles(np.array([0x0A, 0xB0, 0x78], dtype=np.uint8), 6).tolist() == [0xA, 0, 0, 0xB, 8, 7]


def test_nibbles_against_per_element_definition():
    rng = np.random.default_rng(18)
    codes = rng.integers(0, 16, size=4096, dtype=np.uint8)
    packed = oracle.pack_nibbles(codes)
    assert packed.size == codes.size // 2
    for j in range(codes.size):
        byte = int(packed[j // 2])
        assert ((byte >> (4 * (j % 2))) & 0xF) == int(codes[j]), j
    raw = rng.integers(0, 256, size=2048, dtype=np.uint8)
    out = oracle.unpack_nibbles(raw, 2 * raw.size)
    for j in range(out.size):
        want = int(raw[j // 2]) & 0xF if j % 2 == 0 else int(raw[j // 2]) >> 4
        assert int(out[j]) == want, j


def test_pack_bits_hand_written_bytes():
    flags = [1, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 0, 0, 0, 0, 1]
    assert oracle.pack_bits(flags).tolist() == [0x01, 0x82]
    assert oracle.unpack_bits(np.array([0x01, 0x82], dtype=np.uint8), 16).tolist() == flags


def test_capture_record_bytes_by_hand():
    """One block worked by hand.  ts = 1 and block maximum 6 give
    v = fl32(fl32(6 / 6) / 1) = 1, scale byte E4M3FN(1.0) = 0x38 and s = 1,
    so each code is the E2M1 code of the element itself:
    0.5 -> 0x1, -3 -> 0xD, 6 -> 0x7, -0 -> 0x8, 1.5 -> 0x3, then zeros."""
    vals = np.zeros(16, dtype=np.float32)
    vals[:5] = [0.5, -3.0, 6.0, -0.0, 1.5]
    x = (vals.view(np.uint32) >> 16).astype(np.uint16)
    cap = oracle.capture(x, np.float32(1.0), with_codes=True)
    assert cap["scales"].tolist() == [0x38]
    # codes: (x1 << 4 | x0), (x3 << 4 | x2), (x5 << 4 | x4), ...
    assert cap["codes"].tolist() == [0xD1, 0x87, 0x03, 0, 0, 0, 0, 0]
    # parity bits of the indices 1, 5, 7, 0, 3, 0, ...: elements 0, 1, 2 and 4
    assert cap["bits"].tolist() == [0b00010111, 0x00]
