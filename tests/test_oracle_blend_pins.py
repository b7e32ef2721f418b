"""Pins of the oracle's warm-up blend (Hugging Face 1.58-bit write-up, section
"동적 워밍업 양자화": lambda = min(step / total, 1) scales the difference between
the original and the quantised values, so lambda = 0 is the full-precision
layer and lambda = 1 the BitLinear layer).

CPU only.  The end points are pinned to independent computations: lambda = 1
to the oracle's integer contraction and dequantisation (pinned elsewhere to a
matmul of the codes), lambda = 0 to the dense layer written with numpy
(RMSNorm, then a float64 matmul with the full-precision weights).  In between,
the blend of both operands makes y a quadratic in lambda whose coefficients are
the four products of {full precision, dequantised} activations and weights;
that expansion is computed here with numpy matmuls, not with the oracle's loop.
"""
import numpy as np
import pytest

from bit_gemm_ternary_amd import synth


def _layer(M, N, K, seed, gain=False):
    x = synth.activations(M, K, seed, seed + 1, outlier_frac=0.01, outlier_factor=20.0)
    W = synth.weights(N, K, seed + 2)
    g = np.random.default_rng(seed + 3).uniform(0.5, 1.5, K).astype(np.float32) if gain else None
    return x, W, g


def _dense_parts(orc, x, W, g, eps=1e-5):
    """(n, n~, W, W~) in float64 from numpy and the oracle's codes."""
    xf = synth.bf16_to_float(x).astype(np.float64)
    u = synth.bf16_to_float(x) * (g if g is not None else np.float32(1.0))   # float32 product, as O2
    rstd = 1.0 / np.sqrt(np.mean(xf * xf, axis=1) + eps)
    n = u.astype(np.float64) * rstd[:, None]
    q, d_x, _ = orc.quant_act(x, gain=g, eps=eps)
    nt = q.astype(np.float64) * d_x.astype(np.float64)[:, None]
    _, d_w, _, qw = orc.pack_weights(W)
    wt = qw.astype(np.float64) * np.float64(d_w)
    return n, nt, W.astype(np.float64), wt


def test_lambda_schedule(orc):
    assert orc.warmup_lambda(0, 1000) == 0.0
    assert orc.warmup_lambda(-5, 1000) == 0.0
    assert orc.warmup_lambda(250, 1000) == 0.25
    assert orc.warmup_lambda(1000, 1000) == 1.0
    assert orc.warmup_lambda(5000, 1000) == 1.0
    assert orc.warmup_lambda(7, 0) == 1.0


@pytest.mark.parametrize("gain", [False, True])
def test_lambda_one_is_the_bitlinear_layer(orc, gain):
    M, N, K = 3, 40, 256
    x, W, g = _layer(M, N, K, 3100, gain)
    y = orc.linear_forward_blend(x, W, 1.0, gain=g)
    q, d_x, _ = orc.quant_act(x, gain=g)
    packed, d_w, _, _ = orc.pack_weights(W)
    _, want = orc.linear_forward(q, d_x, packed, d_w, K)
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-14 * np.abs(want).max())


@pytest.mark.parametrize("gain", [False, True])
def test_lambda_zero_is_the_dense_layer(orc, gain):
    M, N, K = 4, 33, 192
    x, W, g = _layer(M, N, K, 3200, gain)
    y = orc.linear_forward_blend(x, W, 0.0, gain=g)
    xf = synth.bf16_to_float(x).astype(np.float64)
    gg = np.ones(K) if g is None else g.astype(np.float64)
    n = xf * gg / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + 1e-5)
    want = n @ W.astype(np.float64).T
    # u = float32(x * g) in the oracle: one float32 rounding per product
    np.testing.assert_allclose(y, want, rtol=1e-6, atol=1e-6 * np.abs(want).max())


@pytest.mark.parametrize("lam", [0.25, 0.5, 0.8])
def test_blend_is_quadratic_in_lambda_over_both_operands(orc, lam):
    M, N, K = 5, 48, 256
    x, W, g = _layer(M, N, K, 3300, True)
    n, nt, w, wt = _dense_parts(orc, x, W, g)
    y00, y01, y10, y11 = n @ w.T, n @ wt.T, nt @ w.T, nt @ wt.T
    want = (1 - lam) ** 2 * y00 + lam * (1 - lam) * (y01 + y10) + lam ** 2 * y11
    y = orc.linear_forward_blend(x, W, lam, gain=g)
    np.testing.assert_allclose(y, want, rtol=1e-9, atol=1e-11 * np.abs(want).max())


def test_blend_moves_from_dense_to_ternary_monotonically_in_error(orc):
    # |y(lam) - y(0)| grows with lam on a layer where quantisation changes y
    M, N, K = 2, 64, 512
    x, W, g = _layer(M, N, K, 3400)
    y0 = orc.linear_forward_blend(x, W, 0.0)
    errs = [np.abs(orc.linear_forward_blend(x, W, lam) - y0).mean() for lam in (0.1, 0.4, 0.7, 1.0)]
    assert errs[0] > 0 and all(a < b for a, b in zip(errs, errs[1:]))
