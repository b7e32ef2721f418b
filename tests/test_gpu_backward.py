"""GPU parity of the straight-through-estimator backward against the CPU oracle.

Bars (derived from the arithmetic, written out per test):
* packed transpose: bit-exact.
* grad_n = d_w * grad_y @ q_w: every product grad_y * q (bf16 times -1, 0, 1) is
  exact, so the only rounding is the float32 accumulation of N terms and the
  final scaling: |got - want| <= N 2^-24 d_w sum_n |grad_y q| + 2^-23 |want|.
* grad_w = sum_m grad_y d_x q_x: grad_y * d_x is rounded to float32 and carried
  as bf16 hi + lo (|p - hi - lo| <= 2^-16 |p|), products with the codes are
  exact, and 2 Mp terms (Mp = M rounded up to 64) are accumulated in float32:
  |got - want| <= (2^-16 + 2^-24 + 2 Mp 2^-24) sum_m |grad_y d_x q_x| + 2^-23 |want|.
* RMSNorm backward: the same float64 formula, summed in another order and
  rounded to float32: |got - want| <= 2^-22 (|g r grad_n| + |x r^3 dot / K|).
Elementwise relative error is not meaningful for these sums (they cancel), so
each bound is relative to the sum of the magnitudes of the terms.
"""
import numpy as np
import pytest

import bit_gemm_ternary_amd as bt
from bit_gemm_ternary_amd import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    bt.lib()
    return torch.device("cuda:0")


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_to_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def grad_bits(M, N, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return synth.bf16_bits((rng.standard_normal((M, N)) * scale).astype(np.float32))


def assert_within(got, want, tol, what):
    err = np.abs(np.asarray(got, np.float64) - want)
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} values outside the bound; first at "
                           f"{np.argwhere(bad)[0]}: got {got[bad][0]} want {want[bad][0]} tol {tol[bad][0]}")


def packed_for(orc, N, K, seed, dev):
    packed, d_w, _, q = orc.pack_weights(synth.weights(N, K, seed=seed))
    ws = to_dev(np.array([d_w, 0.0], np.float32), dev)
    return packed, np.float32(d_w), q, to_dev(packed, dev), ws


# ---------------------------------------------------------------------------
# Packed transpose.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K", [(64, 64), (128, 256), (192, 320), (4096, 4096), (11008, 4096),
                                 (4096, 11008), (14336, 4096)])
def test_transpose_packed(orc, dev, N, K):
    packed, _, _, pd, _ = packed_for(orc, N, K, 300 + N % 91, dev)
    got = host(bt.transpose_packed(pd, K))
    want = orc.transpose_packed(packed, K)
    assert np.count_nonzero(got != want) == 0


# ---------------------------------------------------------------------------
# grad_n = d_w * grad_y @ q_w.
# ---------------------------------------------------------------------------

def check_backward_input(orc, g_bits, packed, d_w, q, K, got):
    want = orc.linear_backward_input(g_bits, packed, d_w, K)
    N = g_bits.shape[1]
    mag = np.abs(synth.bf16_to_float(g_bits).astype(np.float64)) @ np.abs(q.astype(np.float64))
    tol = N * U * float(d_w) * mag + 2 * U * np.abs(want)
    assert_within(got, want, tol, "grad_n")


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (5, 128, 256), (300, 192, 320), (64, 4096, 4096),
                                   (33, 11008, 4096), (17, 4096, 11008), (513, 640, 1152)])
def test_linear_backward_input(orc, dev, M, N, K):
    packed, d_w, q, pd, ws = packed_for(orc, N, K, 310 + M, dev)
    g = grad_bits(M, N, 311 + N % 97)
    got = host(bt.linear_backward_input(bf16_to_dev(g, dev), bt.transpose_packed(pd, K), ws))
    check_backward_input(orc, g, packed, d_w, q, K, got)


@pytest.mark.parametrize("N", [4096, 14336])
def test_linear_backward_input_full_size_sampled(orc, dev, N):
    # M 2048 tokens back through N outputs to K 4096 (N 14336: the benchmark's
    # prefill layer), checked on 24 sampled tokens
    M, K = 2048, 4096
    packed, d_w, q, pd, ws = packed_for(orc, N, K, 320, dev)
    g = grad_bits(M, N, 321)
    got = host(bt.linear_backward_input(bf16_to_dev(g, dev), bt.transpose_packed(pd, K), ws))
    rows = np.sort(np.random.default_rng(322).choice(M, 24, replace=False))
    rows[0], rows[-1] = 0, M - 1
    check_backward_input(orc, g[rows], packed, d_w, q, K, got[rows])


def test_linear_backward_input_over_a_million_tokens(orc, dev):
    # more tokens than one launch covers (2^20 rows each): the row ranges must
    # join without a gap; sampled tokens on both sides of the seam
    M, N, K = (1 << 20) + 300, 64, 64
    packed, d_w, q, pd, ws = packed_for(orc, N, K, 323, dev)
    g = grad_bits(M, N, 324)
    got = host(bt.linear_backward_input(bf16_to_dev(g, dev), bt.transpose_packed(pd, K), ws))
    rows = np.array([0, 1, (1 << 20) - 1, 1 << 20, (1 << 20) + 1, M - 1])
    rows = np.concatenate([rows, np.random.default_rng(325).choice(M, 26, replace=False)])
    check_backward_input(orc, g[rows], packed, d_w, q, K, got[rows])


def test_linear_backward_input_empty_batch(dev):
    packed = torch.full((64, 64 // 4), 0x55, dtype=torch.uint8, device=dev)
    out = bt.linear_backward_input(torch.empty((0, 64), dtype=torch.bfloat16, device=dev),
                                   bt.transpose_packed(packed, 64),
                                   torch.ones(2, dtype=torch.float32, device=dev))
    assert tuple(out.shape) == (0, 64)


# ---------------------------------------------------------------------------
# grad_w = sum_m grad_y d_x q_x.
# ---------------------------------------------------------------------------

def codes(M, K, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    d_x = rng.uniform(1e-3, 5e-2, M).astype(np.float32)
    return q, d_x


def check_backward_weight(orc, g_bits, xq, d_x, got):
    want = orc.linear_backward_weight(g_bits, xq, d_x)
    M = g_bits.shape[0]
    Mp = -(-M // 64) * 64
    p = np.abs(synth.bf16_to_float(g_bits).astype(np.float64) * d_x.astype(np.float64)[:, None])
    mag = p.T @ np.abs(xq.astype(np.float64))
    tol = (2.0 ** -16 + U + 2 * Mp * U) * mag + 2 * U * np.abs(want)
    assert_within(got, want, tol, "grad_w")


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (7, 128, 256), (300, 192, 320), (100, 4096, 4096),
                                   (64, 11008, 4096), (65, 4096, 11008), (129, 1088, 704)])
def test_linear_backward_weight(orc, dev, M, N, K):
    xq, d_x = codes(M, K, 330 + M)
    g = grad_bits(M, N, 331 + N % 89)
    got = host(bt.linear_backward_weight(bf16_to_dev(g, dev), to_dev(xq, dev), to_dev(d_x, dev)))
    check_backward_weight(orc, g, xq, d_x, got)


@pytest.mark.parametrize("N", [4096, 14336])
def test_linear_backward_weight_full_size_sampled(orc, dev, N):
    # M 2048 tokens, N outputs, K 4096 (N 14336: the benchmark's prefill
    # layer); sampled 32 x 64 block of grad_w
    M, K = 2048, 4096
    xq, d_x = codes(M, K, 340)
    g = grad_bits(M, N, 341)
    got = host(bt.linear_backward_weight(bf16_to_dev(g, dev), to_dev(xq, dev), to_dev(d_x, dev)))
    rng = np.random.default_rng(342)
    ns = np.sort(rng.choice(N, 32, replace=False))
    ks = np.sort(rng.choice(K, 64, replace=False))
    ns[-1], ks[-1] = N - 1, K - 1
    check_backward_weight(orc, g[:, ns], xq[:, ks], d_x, got[np.ix_(ns, ks)])


def test_linear_backward_weight_at_the_token_limit(orc, dev):
    # 2^21 tokens, the most dL/dW takes: operand rows of 2^22 bf16 values
    M, N, K = 1 << 21, 128, 64
    xq, d_x = codes(M, K, 343)
    g = grad_bits(M, N, 344)
    got = host(bt.linear_backward_weight(bf16_to_dev(g, dev), to_dev(xq, dev), to_dev(d_x, dev)))
    ns, ks = np.array([0, 77, 127]), np.array([0, 31, 63])
    check_backward_weight(orc, g[:, ns], xq[:, ks], d_x, got[np.ix_(ns, ks)])


def test_linear_backward_weight_empty_batch_is_zero(dev):
    out = torch.full((64, 128), 7.0, dtype=torch.float32, device=dev)
    bt.linear_backward_weight(torch.empty((0, 64), dtype=torch.bfloat16, device=dev),
                              torch.empty((0, 128), dtype=torch.int8, device=dev),
                              torch.empty(0, dtype=torch.float32, device=dev), out=out)
    assert (host(out) == 0).all()


# ---------------------------------------------------------------------------
# RMSNorm backward.
# ---------------------------------------------------------------------------

def check_rmsnorm(orc, x_bits, gn, gain, eps, gx, gg):
    want_x, want_g = orc.rmsnorm_backward(x_bits, gn, gain=gain, eps=eps, with_gain_grad=gg is not None)
    x = synth.bf16_to_float(x_bits).astype(np.float64)
    g = np.ones(x.shape[1]) if gain is None else gain.astype(np.float64)
    K = x.shape[1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    dot = np.sum(gn.astype(np.float64) * x * g, axis=1, keepdims=True)
    mag = np.abs(g * r * gn) + np.abs(x * r ** 3 * dot / K)
    assert_within(gx, want_x, 4 * U * mag + 1e-30, "grad_x")
    if gg is not None:
        magg = np.sum(np.abs(gn.astype(np.float64) * x * r), axis=0)
        assert_within(gg, want_g, 2 * U * np.abs(want_g) + 1e-13 * magg + 1e-30, "grad_gain")


@pytest.mark.parametrize("M,K,with_gain", [(1, 64, False), (7, 256, True), (33, 4096, False),
                                           (2048, 4096, True), (3, 14336, True)])
def test_rmsnorm_backward(orc, dev, M, K, with_gain):
    rng = np.random.default_rng(350 + M)
    x_bits = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    gn = rng.standard_normal((M, K)).astype(np.float32)
    gain = rng.uniform(0.5, 1.5, K).astype(np.float32) if with_gain else None
    gx, gg = bt.rmsnorm_backward(bf16_to_dev(x_bits, dev), to_dev(gn, dev),
                                 gain=None if gain is None else to_dev(gain, dev), eps=1e-5,
                                 with_gain_grad=with_gain)
    check_rmsnorm(orc, x_bits, gn, gain, 1e-5, host(gx), None if gg is None else host(gg))


# ---------------------------------------------------------------------------
# The whole STE backward of one BitLinear layer.
# ---------------------------------------------------------------------------

def test_bitlinear_backward_chain(orc, dev):
    M, N, K = 96, 1024, 4096
    W = synth.weights(N, K, seed=360)
    x_bits = synth.activations(M, K, 361, 362, outlier_frac=0.01, outlier_factor=20.0)
    g_bits = grad_bits(M, N, 363, scale=1e-2)
    gain = np.random.default_rng(364).uniform(0.5, 1.5, K).astype(np.float32)
    # oracle: pack, quantise, the two contractions, the RMSNorm backward
    packed, d_w, _, q = orc.pack_weights(W)
    xq, d_x, _ = orc.quant_act(x_bits, gain, 1e-5)
    want_gn = orc.linear_backward_input(g_bits, packed, d_w, K)
    want_gw = orc.linear_backward_weight(g_bits, xq, d_x)
    # GPU: the same chain through the C ABI
    pd, ws = bt.pack_weights(to_dev(W, dev))
    gq, gdx, _ = bt.quant_act(bf16_to_dev(x_bits, dev), to_dev(gain, dev), 1e-5)
    gy = bf16_to_dev(g_bits, dev)
    gn = bt.linear_backward_input(gy, bt.transpose_packed(pd, K), ws)
    gw = bt.linear_backward_weight(gy, gq, gdx)
    gx, gg = bt.rmsnorm_backward(bf16_to_dev(x_bits, dev), gn, gain=to_dev(gain, dev), eps=1e-5,
                                 with_gain_grad=True)
    np.testing.assert_array_equal(host(gq), xq)
    check_backward_input(orc, g_bits, packed, d_w, q, K, host(gn))
    check_backward_weight(orc, g_bits, xq, d_x, host(gw))
    # the RMSNorm backward is checked on the GPU's grad_n (its own input)
    check_rmsnorm(orc, x_bits, host(gn), gain, 1e-5, host(gx), host(gg))
    assert np.all(np.isfinite(want_gn)) and np.all(np.isfinite(want_gw))
