"""Host encoder/decoder of the 6-bit activation layout (xq6) of
bitnet_hadamard_quant_act_f6 / bitnet_linear_forward_f6, written from the
header's description: int4 codes as E3M2 floats, 32 values per 24-byte group,
value p of a group at bits 6p..6p+5 holding the code at K offset
16 (p % 2) + 4 (p / 8) + (p % 8) / 2.  Test infrastructure only."""
import numpy as np

# K offset of value p within a 32-value group
KAPPA = np.array([16 * (p % 2) + 4 * (p // 8) + (p % 8) // 2 for p in range(32)])


def e3m2_of_int(v: np.ndarray) -> np.ndarray:
    v = v.astype(np.int64)
    a = np.abs(v)
    lg = np.zeros_like(a)
    nz = a > 0
    lg[nz] = np.floor(np.log2(a[nz])).astype(np.int64)
    m = ((a << 2) >> lg) & 3
    code = np.where(nz, ((lg + 3) << 2) | m, 0) | np.where(v < 0, 0x20, 0)
    return code.astype(np.uint64)


def int_of_e3m2(code: np.ndarray) -> np.ndarray:
    code = code.astype(np.int64)
    s = (code >> 5) & 1
    e = (code >> 2) & 7
    m = code & 3
    mag = np.where(e == 0, m / 4.0 * 2.0 ** -2, (1 + m / 4.0) * 2.0 ** (e - 3))
    val = np.where(s == 1, -mag, mag)
    assert np.all(val == np.round(val)), "non-integer code"
    return val.astype(np.int64)


def encode(codes: np.ndarray) -> np.ndarray:
    """int codes [M][K] in [-8, 8] -> xq6 bytes [M][K/4*3]."""
    M, K = codes.shape
    g = codes.reshape(M, K // 32, 32)[:, :, KAPPA]          # value p = code at KAPPA[p]
    f = e3m2_of_int(g)                                        # [M][G][32] 6-bit codes
    words = np.zeros((M, K // 32, 3), np.uint64)              # 192 bits as 3 x 64
    for p in range(32):
        bit = 6 * p
        words[:, :, bit // 64] |= (f[:, :, p] << np.uint64(bit % 64)) & np.uint64(0xFFFFFFFFFFFFFFFF)
        if bit % 64 > 58:
            words[:, :, bit // 64 + 1] |= f[:, :, p] >> np.uint64(64 - bit % 64)
    return words.astype("<u8").view(np.uint8).reshape(M, K // 4 * 3)


def decode(xq6: np.ndarray, K: int) -> np.ndarray:
    """xq6 bytes [M][K/4*3] -> int codes [M][K]."""
    M = xq6.shape[0]
    words = np.ascontiguousarray(xq6).view("<u8").reshape(M, K // 32, 3).astype(np.uint64)
    out = np.zeros((M, K // 32, 32), np.int64)
    for p in range(32):
        bit = 6 * p
        v = words[:, :, bit // 64] >> np.uint64(bit % 64)
        if bit % 64 > 58:
            v = v | (words[:, :, bit // 64 + 1] << np.uint64(64 - bit % 64))
        out[:, :, KAPPA[p]] = int_of_e3m2(v & np.uint64(63))
    return out.reshape(M, K)
