"""The host-side packer and unpacker of 6- and 4-bit LeapQuant code rows (used by the
GPU tests to check the stored bytes) pinned to hand-worked bytes and round trips."""
import numpy as np

from helpers import pack_codes, unpack_codes


def test_four_bit_bytes_by_hand():
    z = np.zeros(128, np.int8)
    z[:4] = [1, -1, 7, -7]               # nibbles 0x1, 0xF, 0x7, 0x9
    raw = pack_codes(z, 4)
    assert raw.shape == (64,) and raw[0] == 0xF1 and raw[1] == 0x97 and not raw[2:].any()
    assert np.array_equal(unpack_codes(raw, 4), z)


def test_six_bit_bytes_by_hand():
    z = np.zeros(128, np.int8)
    z[4:8] = [1, -1, 31, -31]            # group 1: 0x01 | 0x3F << 6 | 0x1F << 12 | 0x21 << 18
    word = 0x01 | (0x3F << 6) | (0x1F << 12) | (0x21 << 18)
    raw = pack_codes(z, 6)
    assert raw.shape == (96,) and not raw[:3].any() and not raw[6:].any()
    assert list(raw[3:6]) == [word & 255, (word >> 8) & 255, word >> 16]
    assert np.array_equal(unpack_codes(raw, 6), z)


def test_round_trip_full_range():
    rng = np.random.default_rng(7)
    for bits in (4, 6, 8):
        Q = (1 << (bits - 1)) - 1
        z = rng.integers(-Q, Q + 1, size=(3, 5, 128)).astype(np.int8)
        raw = pack_codes(z, bits)
        assert raw.shape[-1] == (16 * bits if bits < 8 else 128)
        assert np.array_equal(unpack_codes(raw, bits), z)
