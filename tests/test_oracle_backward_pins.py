"""Pins of the oracle's straight-through-estimator backward pass.

CPU only (no ``gpu`` marker).  None of these tests retypes a backward formula.
The contractions are pinned to the forward contraction (itself pinned to an
integer matmul) through the adjoint identity <g, A v> = <A^T g, v>, and by
closed forms; the RMSNorm backward is pinned to central finite differences of
the RMSNorm forward written as its definition, and to the scale invariance
of RMSNorm without epsilon.
"""
import numpy as np

from bit_gemm_ternary_amd import synth


def _grad_bits(M, N, seed):
    rng = np.random.default_rng(seed)
    return synth.bf16_bits(rng.standard_normal((M, N)).astype(np.float32))


def test_transpose_packed_moves_every_field(orc):
    N, K = 48, 80
    packed, _, _, q = orc.pack_weights(synth.weights(N, K, seed=201))
    pt = orc.transpose_packed(packed, K)
    assert pt.shape == (K, N // 4)
    np.testing.assert_array_equal(orc.unpack_weights(pt, N), q.T)
    np.testing.assert_array_equal(orc.transpose_packed(pt, N), packed)


def test_backward_input_is_the_adjoint_of_the_forward(orc):
    # sum_{m,n} g[m,n] (d_w q_x q_w^T)[m,n] == sum_{m,k} q_x[m,k] grad_n[m,k]
    M, N, K = 5, 64, 96
    rng = np.random.default_rng(202)
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    packed, _, _, _ = orc.pack_weights(synth.weights(N, K, seed=203))
    d_w = np.float32(0.0173)
    g = _grad_bits(M, N, 204)
    acc = orc.int_gemm(xq, packed, K).astype(np.float64)
    lhs = float(np.sum(synth.bf16_to_float(g).astype(np.float64) * acc) * np.float64(d_w))
    grad_n = orc.linear_backward_input(g, packed, d_w, K)
    rhs = float(np.sum(xq.astype(np.float64) * grad_n))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_backward_input_closed_forms(orc):
    # all codes +1: every column is d_w * sum_n g[m, n]; one nonzero weight picks one g column
    M, N, K = 3, 32, 64
    g = _grad_bits(M, N, 205)
    gf = synth.bf16_to_float(g).astype(np.float64)
    packed, d_w, _, _ = orc.pack_weights(np.ones((N, K), np.float32))
    grad_n = orc.linear_backward_input(g, packed, d_w, K)
    np.testing.assert_allclose(grad_n, np.repeat(gf.sum(1, keepdims=True) * float(d_w), K, 1), rtol=1e-14)
    W = np.zeros((N, K), np.float32)
    W[7, 11] = -1.0
    packed, d_w, _, _ = orc.pack_weights(W)
    grad_n = orc.linear_backward_input(g, packed, d_w, K)
    want = np.zeros((M, K))
    want[:, 11] = -gf[:, 7] * float(d_w)
    np.testing.assert_array_equal(grad_n, want)


def test_backward_weight_is_the_adjoint_of_the_forward(orc):
    # sum_{n,k} grad_w[n,k] q_w[n,k] == sum_{m,n} g[m,n] d_x[m] (q_x q_w^T)[m,n]
    M, N, K = 6, 40, 128
    rng = np.random.default_rng(206)
    xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    d_x = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    packed, _, _, q = orc.pack_weights(synth.weights(N, K, seed=207))
    g = _grad_bits(M, N, 208)
    grad_w = orc.linear_backward_weight(g, xq, d_x)
    assert grad_w.shape == (N, K)
    lhs = float(np.sum(grad_w * q.astype(np.float64)))
    acc = orc.int_gemm(xq, packed, K).astype(np.float64)
    rhs = float(np.sum(synth.bf16_to_float(g).astype(np.float64) * d_x.astype(np.float64)[:, None] * acc))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs))


def test_backward_weight_single_token_is_an_outer_product(orc):
    N, K = 16, 32
    rng = np.random.default_rng(209)
    xq = rng.integers(-127, 128, size=(1, K)).astype(np.int8)
    d_x = np.array([0.037], np.float32)
    g = _grad_bits(1, N, 210)
    grad_w = orc.linear_backward_weight(g, xq, d_x)
    col = synth.bf16_to_float(g)[0].astype(np.float64) * np.float64(d_x[0])
    np.testing.assert_array_equal(grad_w, np.outer(col, xq[0].astype(np.float64)))


def _rmsnorm(x, gain, eps):
    """n = x * gain / sqrt(mean(x^2) + eps), row-wise, float64."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return x * gain[None, :] * r


def test_rmsnorm_backward_matches_finite_differences(orc):
    M, K, eps = 2, 24, 1e-2
    rng = np.random.default_rng(211)
    x_bits = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    x = synth.bf16_to_float(x_bits).astype(np.float64)
    gain = rng.uniform(0.5, 1.5, K).astype(np.float32)
    gn = rng.standard_normal((M, K)).astype(np.float32)
    grad_x, grad_gain = orc.rmsnorm_backward(x_bits, gn, gain=gain, eps=eps, with_gain_grad=True)
    f = lambda xx, gg: float(np.sum(gn.astype(np.float64) * _rmsnorm(xx, gg, eps)))
    g64 = gain.astype(np.float64)
    h = 1e-6
    num_x = np.zeros((M, K))
    for m in range(M):
        for k in range(K):
            e = np.zeros((M, K))
            e[m, k] = h
            num_x[m, k] = (f(x + e, g64) - f(x - e, g64)) / (2 * h)
    num_g = np.zeros(K)
    for k in range(K):
        e = np.zeros(K)
        e[k] = h
        num_g[k] = (f(x, g64 + e) - f(x, g64 - e)) / (2 * h)
    np.testing.assert_allclose(grad_x, num_x, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(grad_gain, num_g, rtol=1e-6, atol=1e-8)
    gx_nogain, _ = orc.rmsnorm_backward(x_bits, gn, gain=None, eps=eps)
    ones = np.ones(K)
    num_1 = np.array([[(f(x + np.eye(M * K)[m * K + k].reshape(M, K) * h, ones)
                        - f(x - np.eye(M * K)[m * K + k].reshape(M, K) * h, ones)) / (2 * h)
                       for k in range(K)] for m in range(M)])
    np.testing.assert_allclose(gx_nogain, num_1, rtol=1e-6, atol=1e-8)


def test_rmsnorm_backward_is_orthogonal_to_x_without_eps(orc):
    # n(a x) = n(x) for a > 0 when eps = 0, so the gradient has no component along x.
    M, K = 3, 64
    rng = np.random.default_rng(212)
    x_bits = synth.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    x = synth.bf16_to_float(x_bits).astype(np.float64)
    gn = rng.standard_normal((M, K)).astype(np.float32)
    grad_x, _ = orc.rmsnorm_backward(x_bits, gn, gain=rng.uniform(0.5, 1.5, K).astype(np.float32), eps=0.0)
    dots = np.sum(grad_x * x, axis=1)
    assert np.all(np.abs(dots) <= 1e-12 * np.sum(np.abs(grad_x * x), axis=1))
