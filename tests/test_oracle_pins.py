"""Pins of the CPU oracle against what the pages and the mathematics fix.

CPU only (no ``gpu`` marker).  None of these tests retypes the oracle's
formulas: each one checks a worked example printed on the pages, a closed
form, an invariant, a special case with a known exact answer, or a library
routine (numpy integer matmul, scipy's Sylvester Hadamard matrix, math.fsum).
"""
import math

import numpy as np
import pytest
import scipy.linalg

from bit_gemm_ternary_amd import synth
from conftest import read_golden


def _fields(packed):
    """All 2-bit fields of a packed array, as an int array of shape [..., bytes, 4]."""
    p = packed.astype(np.int64)[..., None]
    return (p >> (2 * np.arange(4))) & 3


# ---------------------------------------------------------------------------
# Weights: ternary codes, packing layout, rounding and scale.
# ---------------------------------------------------------------------------

def test_weight_codes_are_ternary_and_fields_valid(orc):
    W = synth.weights(64, 256, seed=11)
    packed, d_w, s_w, q = orc.pack_weights(W)
    assert packed.shape == (64, 64) and packed.dtype == np.uint8
    assert set(np.unique(q)) == {-1, 0, 1}
    assert _fields(packed).max() <= 2
    np.testing.assert_array_equal(orc.unpack_weights(packed, 256), q)
    golden = read_golden("ternary_levels.txt")
    assert sorted(int(v) for v in golden["levels"]) == sorted(np.unique(q).tolist())
    bits = math.log2(len(golden["levels"]))
    assert math.floor(bits * 1e4) / 1e4 == float(golden["log2_3_truncated"])


def test_packed_bytes_by_hand(orc):
    c = np.float32(0.25)
    # q = +1 at k=0 and -1 at k=12, zero elsewhere: byte 0 holds weights 0, 4, 8, 12
    # in bit pairs 0..3 with fields 2, 1, 1, 0 -> 0b00010110 = 0x16; the other
    # bytes hold only zeros (field 1 in every pair) -> 0x55.
    W = np.zeros((1, 16), np.float32)
    W[0, 0], W[0, 12] = c, -c
    packed, _, _, _ = orc.pack_weights(W)
    assert packed.tolist() == [[0x16, 0x55, 0x55, 0x55]]
    # q = -1, 0, +1, +1 at k = 0, 1, 2, 3: each sits in bit pair 0 of bytes 0..3
    # (fields 0, 1, 2, 2 over a background of field 1).
    W = np.zeros((1, 16), np.float32)
    W[0, 0], W[0, 2], W[0, 3] = -c, c, c
    packed, _, _, _ = orc.pack_weights(W)
    assert packed.tolist() == [[0x54, 0x55, 0x56, 0x56]]
    # weight k = 16 + 4*2 + 3 = 27 -> word 1, byte 3 of that word, bit pair 2
    W = np.zeros((1, 32), np.float32)
    W[0, 27] = c
    packed, _, _, _ = orc.pack_weights(W)
    expect = [0x55] * 8
    expect[7] = 0x55 + (1 << 4)
    assert packed.tolist() == [expect]


def test_shift_mask_unpacks_in_natural_order(orc):
    """((word >> 2i) & 0x03030303) yields the codes of weights 16g+4i .. 16g+4i+3 in order."""
    W = synth.weights(8, 512, seed=12)
    packed, _, _, q = orc.pack_weights(W)
    words = packed.view("<u4")  # [N][K/16]
    for i in range(4):
        b = ((words >> np.uint32(2 * i)) & np.uint32(0x03030303)).view(np.uint8)  # [N][K/4]
        got = b.reshape(8, -1, 4).astype(np.int16) - 1          # [N][word][byte]
        want = q.reshape(8, -1, 4, 4)[:, :, i, :]               # [N][word][slot i][byte]
        np.testing.assert_array_equal(got, want)


def test_pack_unpack_round_trip(orc):
    rng = np.random.default_rng(13)
    fields = rng.integers(0, 3, size=(32, 128 // 4, 4))
    packed = (fields << (2 * np.arange(4))).sum(-1).astype(np.uint8)
    q = orc.unpack_weights(packed, 128)
    assert set(np.unique(q)) <= {-1, 0, 1}
    # A ternary matrix is its own quantisation (every nonzero has magnitude 1 and
    # the mean magnitude is <= 1, so scaling then clamping gives it back).
    repacked, _, _, q2 = orc.pack_weights(q.astype(np.float32))
    np.testing.assert_array_equal(repacked, packed)
    np.testing.assert_array_equal(q2, q)


def test_round_half_even_and_clamp(orc):
    e25, e24 = np.float32(2.0 ** -25), np.float32(2.0 ** -24)
    half = np.float32(0.5)
    W = np.array([[0.5, -0.5, 1.5, -1.5, half - e25, -(half - e25), half + e24, -(half + e24),
                   2.5, -2.5, 1, 1, 1, 1, 1 - e24, 0]], np.float32)
    assert math.fsum(np.abs(W.astype(np.float64)).ravel()) == 16.0  # mean |W| = 1 exactly
    packed, d_w, s_w, q = orc.pack_weights(W)
    assert s_w == 1.0 and d_w == 1.0
    assert q[0].tolist() == [0, 0, 1, -1, 0, 0, 1, -1, 1, -1, 1, 1, 1, 1, 1, 0]


def test_absmean_scale_against_exact_sum(orc):
    W = synth.weights(96, 320, seed=14)
    _, d_w, s_w, _ = orc.pack_weights(W)
    mean = math.fsum(np.abs(W.astype(np.float64)).ravel()) / W.size
    assert abs(float(d_w) - mean) <= 1e-7 * mean
    assert abs(float(s_w) - 1.0 / mean) <= 1e-7 / mean
    # and scale 0 for an all-zero matrix: every code 0, packed bytes 0x55
    packed, d0, s0, q0 = orc.pack_weights(np.zeros((3, 64), np.float32))
    assert d0 == 0 and s0 == 0 and not q0.any() and (packed == 0x55).all()


def test_zero_code_fraction_of_gaussian_weights(orc):
    """N(0, s^2) weights scaled by 1/mean|W| are N(0, pi/2): P(|v| < 1/2) = erf(1/(2 sqrt(pi)))."""
    W = synth.weights(512, 1024, seed=15)
    _, _, _, q = orc.pack_weights(W)
    p0 = math.erf(0.5 / math.sqrt(math.pi))
    n = q.size
    tol = 5 * math.sqrt(p0 * (1 - p0) / n)
    assert abs(np.mean(q == 0) - p0) < tol
    assert abs(np.mean(q == 1) - (1 - p0) / 2) < tol
    assert abs(np.mean(q == -1) - (1 - p0) / 2) < tol


def test_hadamard_prerotation_of_scaled_identity(orc):
    """W = c*I rotates to c*H: codes are exactly Sylvester's H, scales c and c/sqrt(K)."""
    K = 256
    c = np.float32(0.125)
    W = (c * np.eye(K)).astype(np.float32)
    packed, d_w, s_w, q = orc.pack_weights(W, hadamard=True)
    np.testing.assert_array_equal(q, scipy.linalg.hadamard(K))
    assert s_w == 8.0 and d_w == np.float32(0.125 / 16)


# ---------------------------------------------------------------------------
# Walsh-Hadamard transform.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64, 256, 1024])
def test_fwht_equals_explicit_sylvester_matrix(orc, n):
    rng = np.random.default_rng(n)
    v = rng.integers(-4, 5, size=(3, n)).astype(np.float32)   # sums stay exact in float32
    H = scipy.linalg.hadamard(n).astype(np.float64)
    np.testing.assert_array_equal(orc.fwht_f32(v).astype(np.float64), v.astype(np.float64) @ H.T)


@pytest.mark.parametrize("n", [2, 16, 128, 512])
def test_fwht_is_a_hadamard_matrix(orc, n):
    H = orc.fwht_f32(np.eye(n, dtype=np.float32)).astype(np.float64)  # rows: transforms of e_j
    np.testing.assert_array_equal(H, H.T)
    np.testing.assert_array_equal(H @ H.T, n * np.eye(n))
    np.testing.assert_array_equal(H[0], np.ones(n))
    assert set(np.unique(H)) == {-1.0, 1.0}


def test_fwht_involution_and_parseval(orc):
    rng = np.random.default_rng(21)
    v = rng.integers(-50, 51, size=(4, 1024)).astype(np.float32)
    np.testing.assert_array_equal(orc.fwht_f32(orc.fwht_f32(v)), 1024 * v)
    x = rng.standard_normal((4, 4096)).astype(np.float32)
    t = orc.fwht_f32(x).astype(np.float64)
    np.testing.assert_allclose((t ** 2).sum(1), 4096 * (x.astype(np.float64) ** 2).sum(1), rtol=1e-5)


# ---------------------------------------------------------------------------
# Activations: int8 absmax codes.
# ---------------------------------------------------------------------------

def _check_absmax_codes(q, u, top):
    """Invariants of absmax codes q of values u (per row) with top code ``top``."""
    u = u.astype(np.float64)
    a = np.abs(u).max(1)
    assert q.min() >= -top and q.max() <= top  # -128 / -8 are never produced
    arg = np.abs(u).argmax(1)
    np.testing.assert_array_equal(np.abs(q[np.arange(len(q)), arg]), top)
    np.testing.assert_array_equal(q[np.arange(len(q)), arg], np.sign(u[np.arange(len(q)), arg]) * top)
    assert ((np.sign(q) == np.sign(u)) | (q == 0)).all()
    exact = top * u / a[:, None]
    assert np.abs(q - exact).max() <= 0.5 + 1e-4
    for r in range(len(q)):  # monotone in u
        order = np.argsort(u[r], kind="stable")
        assert (np.diff(q[r][order].astype(np.int64)) >= 0).all()


def test_int8_codes_invariants(orc):
    x = synth.activations(16, 512, seed=31, outlier_seed=32, outlier_frac=0.01, outlier_factor=20.0)
    q, d_x, qsum = orc.quant_act(x, eps=1e-5)
    u = synth.bf16_to_float(x)
    _check_absmax_codes(q, u, 127)
    np.testing.assert_array_equal(qsum, q.astype(np.int64).sum(1))
    ms = (u.astype(np.float64) ** 2).mean(1)
    want = np.abs(u).max(1) / np.sqrt(ms + 1e-5) / 127
    np.testing.assert_allclose(d_x, want, rtol=1e-7)


def test_int8_codes_power_of_two_invariance(orc):
    x = synth.activations(8, 256, seed=33)
    u = synth.bf16_to_float(x)
    q0, d0, _ = orc.quant_act(x, eps=0.0)
    for j in (-3, 1, 5):
        xj = synth.bf16_bits(u * np.float32(2.0 ** j))   # exact: power-of-two scaling
        qj, dj, _ = orc.quant_act(xj, eps=0.0)
        np.testing.assert_array_equal(qj, q0)
        np.testing.assert_allclose(dj, d0, rtol=1e-6)  # rstd scales inversely


def test_int8_codes_ties_round_to_even(orc):
    vals = np.zeros((1, 64), np.float32)
    vals[0, :5] = [127.0, 2.5, 3.5, -2.5, -3.5]   # absmax 127: factor 127/127 = 1 exactly
    q, _, qsum = orc.quant_act(synth.bf16_bits(vals))
    assert q[0, :5].tolist() == [127, 2, 4, -2, -4]
    assert qsum[0] == 127


def test_int8_gain_is_per_channel(orc):
    x = synth.activations(6, 256, seed=34)
    q0, _, _ = orc.quant_act(x)
    qg, _, _ = orc.quant_act(x, gain=np.full(256, 0.25, np.float32))
    np.testing.assert_array_equal(qg, q0)
    gain = np.ones(256, np.float32)
    gain[17] = 0
    qz, _, _ = orc.quant_act(x, gain=gain)
    assert (qz[:, 17] == 0).all()
    perm = np.random.default_rng(35).permutation(256)
    g = np.random.default_rng(36).uniform(0.5, 1.5, 256).astype(np.float32)
    qa, da, _ = orc.quant_act(x, gain=g)
    qb, db, _ = orc.quant_act(x[:, perm], gain=g[perm])
    np.testing.assert_array_equal(qb, qa[:, perm])
    np.testing.assert_array_equal(db, da)


def test_absmax_worked_example(orc):
    """The primer's example: absmax 5.4, factor 127/5.4 (printed 23.5), divide to dequantise."""
    golden = read_golden("absmax_example.txt")
    absmax = np.float32(golden["absmax"])
    K = 64
    x = synth.bf16_bits(np.ones((1, K), np.float32))        # RMS exactly 1 with eps = 0
    gain = np.zeros(K, np.float32)
    gain[:4] = [absmax, -absmax, 1.0, 2.0]
    q, d_x, _ = orc.quant_act(x, gain=gain, eps=0.0)
    factor = 1.0 / float(d_x[0])
    assert f"{factor:.1f}" == golden["factor_one_decimal"]
    top = int(golden["int8_top"])
    assert q[0, :4].tolist() == [top, -top, 24, 47]           # 23.518 -> 24, 47.037 -> 47
    np.testing.assert_allclose(q[0, :4] * d_x[0], gain[:4], atol=0.5 * float(d_x[0]))


def test_zero_and_tiny_tokens(orc):
    x = np.zeros((3, 128), np.float32)
    x[1, 5] = 2.0 ** -126                  # below the 2^-120 all-zero threshold
    x[2, 9] = 2.0 ** -100
    q, d_x, qsum = orc.quant_act(synth.bf16_bits(x))
    assert not q[:2].any() and d_x[0] == 0 and d_x[1] == 0 and qsum[0] == 0 and qsum[1] == 0
    assert q[2, 9] == 127 and d_x[2] > 0
    qh, dh, sh = orc.hadamard_quant_act(synth.bf16_bits(x))
    assert not qh[:2].any() and dh[0] == 0 and dh[1] == 0 and sh[0] == 0
    assert (np.abs(qh[2]) == 7).all()      # a single spike transforms to +-a everywhere


def test_folded_rstd_changes_only_near_ties(orc):
    """Codes from u vs from u/rms: identical in exact arithmetic; rounding differs rarely."""
    x = synth.activations(64, 1024, seed=37, outlier_seed=38, outlier_frac=0.01, outlier_factor=20.0)
    q, _, _ = orc.quant_act(x, eps=1e-5)
    u = synth.bf16_to_float(x).astype(np.float64)
    xn = u / np.sqrt((u ** 2).mean(1, keepdims=True) + 1e-5)
    v = xn * 127 / np.abs(xn).max(1, keepdims=True)
    literal = np.clip(np.rint(v), -128, 127)
    differ = literal != q
    # The two orders agree except where the exact value is a rounding tie (the
    # float64 literal lands within 1e-9 of a half-integer): there the folded
    # float32 product and the float64 quotient may round to the two neighbours.
    assert differ.sum() <= 4                           # 2 of 65536 at this seed
    assert (np.abs(literal[differ] - q[differ]) == 1).all()
    frac = v[differ] - np.floor(v[differ])
    assert (np.abs(frac - 0.5) < 1e-9).all()


# ---------------------------------------------------------------------------
# Activations: Hadamard + int4 codes.
# ---------------------------------------------------------------------------

def test_int4_codes_invariants(orc):
    K = 1024
    x = synth.activations(12, K, seed=41, dist="student_t")
    q, d_x, qsum = orc.hadamard_quant_act(x, eps=1e-5)
    u = synth.bf16_to_float(x).astype(np.float64)
    t = u @ scipy.linalg.hadamard(K).T.astype(np.float64)
    # float32 butterflies vs the float64 matrix product: compare away from ties only
    _check_absmax_codes_near(q, t, 7)
    np.testing.assert_array_equal(qsum, q.astype(np.int64).sum(1))
    rstd = 1 / np.sqrt((u ** 2).mean(1) + 1e-5)
    np.testing.assert_allclose(d_x, np.abs(t).max(1) * rstd / (7 * math.sqrt(K)), rtol=1e-6)


def _check_absmax_codes_near(q, t, top):
    a = np.abs(t).max(1, keepdims=True)
    assert q.min() >= -top and q.max() <= top
    arg = np.abs(t).argmax(1)
    np.testing.assert_array_equal(np.abs(q[np.arange(len(q)), arg]), top)
    assert np.abs(q - top * t / a).max() <= 0.5 + 1e-3


def test_int4_codes_exact_on_small_integers(orc):
    K = 512
    rng = np.random.default_rng(42)
    v = rng.integers(-3, 4, size=(5, K)).astype(np.float32)
    q, _, _ = orc.hadamard_quant_act(synth.bf16_bits(v))
    t = v.astype(np.float64) @ scipy.linalg.hadamard(K).T    # exact in float32 too
    _check_absmax_codes(q, t, 7)


def test_hadamard_spreads_outliers(orc):
    """Heavy-tailed tokens: the transform lowers absmax/RMS (the variant's purpose)."""
    K = 4096
    x = synth.activations(32, K, seed=43, dist="student_t")
    u = synth.bf16_to_float(x).astype(np.float64)
    t = orc.fwht_f32(synth.bf16_to_float(x)).astype(np.float64)
    ratio = lambda a: (np.abs(a).max(1) / np.sqrt((a ** 2).mean(1))).mean()
    assert ratio(t) < 0.5 * ratio(u)
    assert ratio(t) < 5.0   # Gaussian-like: the max of 4096 normals is ~3.5-4 sigma


# ---------------------------------------------------------------------------
# Integer contraction and dequantisation.
# ---------------------------------------------------------------------------

def test_int_gemm_matches_integer_matmul(orc):
    rng = np.random.default_rng(51)
    M, N, K = 7, 45, 320
    xq = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    W = synth.weights(N, K, seed=52)
    packed, _, _, q = orc.pack_weights(W)
    acc = orc.int_gemm(xq, packed, K)
    np.testing.assert_array_equal(acc, xq.astype(np.int64) @ q.astype(np.int64).T)
    rows, cols = rng.integers(0, M, 50), rng.integers(0, N, 50)
    np.testing.assert_array_equal(orc.int_gemm_sampled(xq, packed, K, rows, cols), acc[rows, cols])


def test_int_gemm_all_ones_and_extremes(orc):
    K = 16384
    ones = np.ones((3, K), np.float32)
    packed, _, _, _ = orc.pack_weights(ones)
    xq = np.full((2, K), -128, np.int8)
    xq[1] = 127
    acc = orc.int_gemm(xq, packed, K)
    assert acc.tolist() == [[-128 * K] * 3, [127 * K] * 3]


def test_dequant_closed_form(orc):
    rng = np.random.default_rng(53)
    acc = rng.integers(-2 ** 20, 2 ** 20, size=(4, 9)).astype(np.int32)
    acc[0, 0] = 0
    d_x = rng.uniform(1e-4, 1e-2, 4).astype(np.float32)
    d_w = np.float32(0.0123)
    y = orc.dequant(acc, d_x, d_w)
    assert y[0, 0] == 0.0
    np.testing.assert_allclose(y, acc * d_x.astype(np.float64)[:, None] * np.float64(d_w), rtol=1e-15)
    assert (np.sign(y) == np.sign(acc)).all()


def test_int8_path_end_to_end_scale(orc):
    """W = c * (random signs): quantisation of W is exact, so y - W.rmsnorm(x) is activation rounding only."""
    M, N, K = 32, 64, 512
    rng = np.random.default_rng(54)
    c = np.float32(0.03125)
    S = rng.choice(np.array([-1.0, 1.0], np.float32), size=(N, K))
    packed, d_w, _, _ = orc.pack_weights(c * S)
    assert d_w == c
    x = synth.activations(M, K, seed=55)
    q, d_x, _ = orc.quant_act(x, eps=1e-5)
    _, y = orc.linear_forward(q, d_x, packed, d_w, K)
    u = synth.bf16_to_float(x).astype(np.float64)
    rstd = 1 / np.sqrt((u ** 2).mean(1, keepdims=True) + 1e-5)
    ref = (u * rstd) @ (c * S.astype(np.float64)).T
    a = np.abs(u).max(1, keepdims=True)
    bound = float(c) * rstd * K * a / 254 * 1.001
    assert (np.abs(y - ref) <= bound).all()
    slope = (y * ref).sum() / (ref * ref).sum()
    assert abs(slope - 1) < 2e-3      # a 127-vs-128 slip would bias this by 0.8%


def test_hadamard_path_end_to_end_scale(orc):
    """W = c*I through the H path: ||y - c*rmsnorm(x)||_2 <= c*rstd*absmax(Hx)/14 per token."""
    K = 256
    c = np.float32(0.125)
    packed, d_w, _, _ = orc.pack_weights((c * np.eye(K)).astype(np.float32), hadamard=True)
    x = synth.activations(16, K, seed=56, dist="student_t")
    q, d_x, _ = orc.hadamard_quant_act(x, eps=1e-5)
    _, y = orc.linear_forward(q, d_x, packed, d_w, K)
    u = synth.bf16_to_float(x).astype(np.float64)
    rstd = 1 / np.sqrt((u ** 2).mean(1) + 1e-5)
    t = u @ scipy.linalg.hadamard(K).T
    err = np.linalg.norm(y - float(c) * u * rstd[:, None], axis=1)
    bound = float(c) * rstd * np.abs(t).max(1) / 14
    assert (err <= bound * 1.01).all()
    assert (err >= bound * 0.05).all()   # and the rounding is real, not skipped


def test_packing_ratio_matches_page(orc):
    g = read_golden("packing_ratio.txt")
    W = synth.weights(8, 128, seed=57)
    packed, _, _, _ = orc.pack_weights(W)
    per_byte = W.size / packed.size
    assert per_byte == 4
    h, layers, vocab = int(g["hidden"]), int(g["layers"]), int(g["vocab"])
    proj = sum(K * N for _, K, N in synth.BLOCK_LAYERS) * layers
    embed = 2 * vocab * h
    before = (proj + embed) / 1e9
    after = (proj / per_byte + embed) / 1e9
    assert round(before) == int(g["params_before_billion"])
    assert f"{after:.1f}" == g["params_after_billion_one_decimal"]
