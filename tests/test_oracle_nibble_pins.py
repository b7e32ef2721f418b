"""Pins of the oracle's packed int4 storage (two activation codes per byte).

CPU only.  The BitNet v2 summary ("초저용량 LLM의 진화: BitNet v2 파헤치기",
section 방법론) quantises the Hadamard-transformed activations to 4 bits, so
two codes fit one byte.  The pages fix no byte layout; the one pinned here is
natural order, 4-bit two's complement, code 2j in the low nibble of byte j.
The pins fix that layout by hand-computed bytes, check that the map from a
code pair to a byte is a bijection onto 0..255, decode the sign with a formula
other than the oracle's, and tie the format to the oracle's H-path codes.
"""
import itertools

import numpy as np
import pytest

from bit_gemm_ternary_amd import synth


def test_hand_computed_bytes(orc):
    # (-8, 7) -> 0x8 | 0x7 << 4; (-1, 0) -> 0xF; (3, -3) -> 0x3 | 0xD << 4
    q = np.array([[-8, 7, -1, 0, 3, -3, 0, 0]], np.int8)
    np.testing.assert_array_equal(orc.pack_nibbles(q), [[0x78, 0x0F, 0xD3, 0x00]])
    np.testing.assert_array_equal(orc.pack_nibbles(np.array([[1, 0], [0, 1]], np.int8)), [[0x01], [0x10]])


def test_code_pairs_to_a_byte_is_a_bijection(orc):
    pairs = np.array(list(itertools.product(range(-8, 8), repeat=2)), np.int8)   # 256 rows of 2
    b = orc.pack_nibbles(pairs)[:, 0].astype(int)
    assert sorted(b.tolist()) == list(range(256))
    np.testing.assert_array_equal(orc.unpack_nibbles(orc.pack_nibbles(pairs)), pairs)


def test_unpack_against_a_sign_extension_formula(orc):
    allb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = orc.unpack_nibbles(allb).astype(int)
    lo, hi = allb[0].astype(int) & 15, allb[0].astype(int) >> 4
    np.testing.assert_array_equal(q[0, 0::2], (lo ^ 8) - 8)
    np.testing.assert_array_equal(q[0, 1::2], (hi ^ 8) - 8)


def _rejected(orc, q):
    try:
        orc.pack_nibbles(q)
    except ValueError:
        return True
    return False


def test_codes_outside_int4_are_rejected(orc):
    for bad in (8, -9, 127):
        q = np.zeros((1, 4), np.int8)
        q[0, 3] = bad
        assert _rejected(orc, q), bad
    assert _rejected(orc, np.zeros((1, 3), np.int8))
    assert not _rejected(orc, np.full((1, 4), -8, np.int8))


@pytest.mark.parametrize("M,K", [(3, 256), (2, 4096)])
def test_hadamard_codes_round_trip(orc, M, K):
    x = synth.activations(M, K, 71, 72, outlier_frac=0.01, outlier_factor=20.0)
    q, _, qsum = orc.hadamard_quant_act(x)
    p = orc.pack_nibbles(q)
    assert p.shape == (M, K // 2)
    np.testing.assert_array_equal(orc.unpack_nibbles(p), q)
    # the code sum read back from the bytes
    np.testing.assert_array_equal(orc.unpack_nibbles(p).astype(np.int64).sum(axis=1), qsum)
