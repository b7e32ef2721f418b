"""Pins of the oracle's base-3 packing (five ternary weights per byte).

CPU only (no ``gpu`` marker).  A ternary weight carries log2 3 = 1.585 bits
(the primer on 1.58-bit quantisation, section "1.58비트는 어디서 나온거에요?"),
and 3^5 = 243 <= 256, so five weights fit one byte at 1.6 bits each.  The pins
below fix the digit order and the offset by hand-computed bytes, check that the
map from five digits to a byte is a bijection onto 0..242, and tie the format to
the 2-bit packing through the codes both hold.
"""
import itertools
import math

import numpy as np
import pytest

from bit_gemm_ternary_amd import synth


def test_hand_computed_bytes(orc):
    # digits c = q + 1 with weight 5j + i at place 3^i
    q = np.array([[1, -1, 0, 0, 1, 1]], np.int8)
    np.testing.assert_array_equal(orc.pack_base3(q, 2), [[2 + 0 + 9 + 27 + 162, 2]])
    assert orc.pack_base3(np.full((1, 5), -1, np.int8), 1)[0, 0] == 0
    assert orc.pack_base3(np.full((1, 5), 1, np.int8), 1)[0, 0] == 242
    for i in range(5):
        q = np.full((1, 5), -1, np.int8)
        q[0, i] = 1
        assert orc.pack_base3(q, 1)[0, 0] == 2 * 3 ** i
        q[0, i] = 0
        assert orc.pack_base3(q, 1)[0, 0] == 3 ** i


def test_five_digits_to_a_byte_is_a_bijection(orc):
    combos = np.array(list(itertools.product((-1, 0, 1), repeat=5)), np.int8)   # 243 rows of 5
    bytes_ = orc.pack_base3(combos, 1)[:, 0].astype(int)
    assert sorted(bytes_.tolist()) == list(range(243))
    back, bad = orc.unpack_base3(orc.pack_base3(combos, 1), 5)
    assert bad == 0
    np.testing.assert_array_equal(back, combos)


@pytest.mark.parametrize("N,K,row_bytes", [(3, 64, 13), (5, 4096, 832), (2, 11008, 2208), (4, 333, 80)])
def test_round_trip_and_padding(orc, N, K, row_bytes):
    rng = np.random.default_rng(K)
    q = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    p3 = orc.pack_base3(q, row_bytes)
    assert p3.max() <= 242
    used = (K + 4) // 5
    assert not p3[:, used:].any()                      # bytes past ceil(K/5) are zero
    if K % 5:                                          # weights past K count as digit 0
        assert p3[:, used - 1].max() < 3 ** (K % 5)
    back, bad = orc.unpack_base3(p3, K)
    assert bad == 0
    np.testing.assert_array_equal(back, q)


def test_same_codes_as_the_two_bit_packing(orc):
    N, K = 16, 320
    packed, _, _, q = orc.pack_weights(synth.weights(N, K, seed=501))
    p3 = orc.pack_base3(orc.unpack_weights(packed, K), 64)
    back, _ = orc.unpack_base3(p3, K)
    np.testing.assert_array_equal(back, q)


def test_density():
    # 1.6 bits per weight against log2 3 = 1.585 and the 2-bit layout's 2
    assert 8 / 5 - math.log2(3) < 0.016
    assert (4096 + 4) // 5 / (4096 // 4) == pytest.approx(0.80, abs=0.001)


def test_rejects_a_code_outside_the_three_levels(orc):
    with pytest.raises(ValueError):
        orc.pack_base3(np.array([[0, 2, 0, 0, 0]], np.int8), 1)
    with pytest.raises(ValueError):
        orc.pack_base3(np.zeros((1, 11), np.int8), 2)    # 11 weights need 3 bytes
