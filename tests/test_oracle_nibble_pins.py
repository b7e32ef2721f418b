"""Pins of the oracle's packed int4 storage (two activation codes per byte).

CPU only.  The BitNet v2 summary ("초저용량 LLM의 진화: BitNet v2 파헤치기",
section 방법론) quantises the Hadamard-transformed activations to 4 bits, so
two codes fit one byte.  The pages fix no byte layout; the one pinned here
packs each group of 16 codes into 8 bytes with code 16g + j in the low nibble
and code 16g + 8 + j in the high nibble of byte 8g + j (4-bit two's
complement), the slot order of the 2-bit weight packing.  The pins fix that
layout by hand-computed bytes and by single-code positions, check that the map
from a code pair to a byte is a bijection onto 0..255, decode the sign with a
formula other than the oracle's, and tie the format to the oracle's H-path
codes.
"""
import itertools

import numpy as np

from bit_gemm_ternary_amd import synth


def test_hand_computed_bytes(orc):
    # byte j = (c_j & 15) | (c_{8+j} & 15) << 4; -8 -> 8, -7 -> 9, -4 -> 0xC, -3 -> 0xD, -2 -> 0xE, -1 -> 0xF
    q = np.array([[-8, 7, -1, 0, 3, -3, 1, 2, 5, -2, 0, 4, -7, 6, -4, 1]], np.int8)
    np.testing.assert_array_equal(orc.pack_nibbles(q), [[0x58, 0xE7, 0x0F, 0x40, 0x93, 0x6D, 0xC1, 0x12]])


def test_single_code_positions(orc):
    # a lone code 1 at K index p lands in byte 8 (p // 16) + p % 8, low nibble
    # for p % 16 < 8, high nibble otherwise
    K = 32
    for p in range(K):
        q = np.zeros((1, K), np.int8)
        q[0, p] = 1
        want = np.zeros(K // 2, np.uint8)
        want[8 * (p // 16) + p % 8] = 0x01 if p % 16 < 8 else 0x10
        np.testing.assert_array_equal(orc.pack_nibbles(q)[0], want, err_msg=f"p={p}")
        np.testing.assert_array_equal(orc.unpack_nibbles(want[None, :]), q)


def test_code_pairs_to_a_byte_is_a_bijection(orc):
    pairs = list(itertools.product(range(-8, 8), repeat=2))
    q = np.zeros((256, 16), np.int8)
    for r, (lo, hi) in enumerate(pairs):
        q[r, 3], q[r, 11] = lo, hi
    p = orc.pack_nibbles(q)
    assert sorted(p[:, 3].astype(int).tolist()) == list(range(256))
    assert not np.delete(p, 3, axis=1).any()
    np.testing.assert_array_equal(orc.unpack_nibbles(p), q)


def test_unpack_against_a_sign_extension_formula(orc):
    b = np.zeros((256, 8), np.uint8)
    b[:, 5] = np.arange(256)
    q = orc.unpack_nibbles(b).astype(int)
    lo, hi = np.arange(256) & 15, np.arange(256) >> 4
    np.testing.assert_array_equal(q[:, 5], (lo ^ 8) - 8)
    np.testing.assert_array_equal(q[:, 13], (hi ^ 8) - 8)
    assert not np.delete(q, [5, 13], axis=1).any()


def _rejected(orc, q):
    try:
        orc.pack_nibbles(q)
    except ValueError:
        return True
    return False


def test_codes_outside_int4_are_rejected(orc):
    for bad in (8, -9, 127):
        q = np.zeros((1, 16), np.int8)
        q[0, 13] = bad
        assert _rejected(orc, q), bad
    assert _rejected(orc, np.zeros((1, 24), np.int8))       # K not a multiple of 16
    assert not _rejected(orc, np.full((1, 16), -8, np.int8))


def test_hadamard_codes_round_trip(orc):
    for M, K in ((3, 256), (2, 4096)):
        x = synth.activations(M, K, 71, 72, outlier_frac=0.01, outlier_factor=20.0)
        q, _, qsum = orc.hadamard_quant_act(x)
        p = orc.pack_nibbles(q)
        assert p.shape == (M, K // 2)
        back = orc.unpack_nibbles(p)
        np.testing.assert_array_equal(back, q)
        np.testing.assert_array_equal(back.astype(np.int64).sum(axis=1), qsum)
