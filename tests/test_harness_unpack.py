"""The parity harness's unpacking of 4-bit value codes (two a byte, element 2i
in the low half of byte i, two's complement), checked on hand-made bytes."""
import numpy as np


def test_unpack_int4_by_hand():
    from hkv_harness import unpack_int4
    # 0x7F: low 0xF = -1, high 0x7 = 7; 0x81: low 1, high 0x8 = -8; 0x00: 0, 0; 0xE9: low 9 = -7, high 0xE = -2
    packed = np.array([[0x7F, 0x81, 0x00, 0xE9]], np.uint8)
    assert unpack_int4(packed).tolist() == [[-1, 7, 1, -8, 0, 0, -7, -2]]


def test_unpack_int4_round_trip():
    from hkv_harness import unpack_int4
    rng = np.random.default_rng(5)
    codes = rng.integers(-7, 8, size=(3, 5, 16)).astype(np.int8)
    packed = ((codes[..., 0::2].astype(np.uint8) & 0xF) | ((codes[..., 1::2].astype(np.uint8) & 0xF) << 4))
    np.testing.assert_array_equal(unpack_int4(packed), codes)
