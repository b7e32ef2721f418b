"""The host encoder/decoder of the 6-bit activation layout, pinned to the E3M2
definition (sign, 3 exponent bits with bias 3, 2 mantissa bits) and to the
layout the header states.  CPU only."""
import numpy as np

import f6_layout


def test_e3m2_holds_every_int4_code_exactly():
    v = np.arange(-8, 9)
    np.testing.assert_array_equal(f6_layout.int_of_e3m2(f6_layout.e3m2_of_int(v)), v)


def test_e3m2_bit_patterns():
    # (1 + m/4) * 2^(e - 3): 1 = e3 m0, 3 = 1.5 * 2 (e4 m2), 5 = 1.25 * 4 (e5 m1),
    # 7 = 1.75 * 4 (e5 m3), 8 = 2^3 (e6 m0); the sign is bit 5
    assert list(f6_layout.e3m2_of_int(np.array([0, 1, 3, 5, 7, -8]))) == [
        0, 0b001100, 0b010010, 0b010101, 0b010111, 0b111000]


def test_group_order_is_a_permutation_and_first_values():
    assert sorted(f6_layout.KAPPA.tolist()) == list(range(32))
    # value p -> K offset 16 (p % 2) + 4 (p / 8) + (p % 8) / 2
    assert f6_layout.KAPPA[:10].tolist() == [0, 16, 1, 17, 2, 18, 3, 19, 4, 20]


def test_encode_places_fields_at_6p():
    codes = np.zeros((1, 32), np.int64)
    codes[0, 17] = 1            # K offset 17 is value p = 3 -> bits 18..23
    b = f6_layout.encode(codes)
    word = int.from_bytes(bytes(b[0]), "little")
    assert word == 0b001100 << 18


def test_roundtrip_random():
    rng = np.random.default_rng(0)
    c = rng.integers(-8, 8, (7, 1024))
    np.testing.assert_array_equal(f6_layout.decode(f6_layout.encode(c), 1024), c)
