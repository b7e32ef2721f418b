"""GPU parity of the warm-up blend (bitnet_linear_forward_blend) against the
oracle's float64 definition.

Tolerance from the arithmetic: each blended operand is a few float32 roundings
from its float64 value (d_x itself a few float32 ulps, as for every
quantisation path), so each product is within ~8 u of a_k b_k, and a float32
sum of K products in any order adds at most (K - 1) u sum_k |a_k b_k|
(u = 2^-24).  The test allows (K + 16) u sum_k |a_k| |b_k| per output, with
|a|, |b| the oracle's operands; the typical error is far below that.
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


def _bound(orc, x, W, g, lam, K, eps=1e-5):
    xf = synth.bf16_to_float(x).astype(np.float64)
    u = synth.bf16_to_float(x) * (g if g is not None else np.float32(1.0))
    rstd = 1.0 / np.sqrt(np.mean(xf * xf, axis=1) + eps)
    n = u.astype(np.float64) * rstd[:, None]
    q, d_x, _ = orc.quant_act(x, gain=g, eps=eps)
    nt = q.astype(np.float64) * d_x.astype(np.float64)[:, None]
    _, d_w, _, qw = orc.pack_weights(W)
    w = W.astype(np.float64)
    wt = qw.astype(np.float64) * np.float64(d_w)
    a = n + lam * (nt - n)
    b = w + lam * (wt - w)
    return (K + 16) * U * (np.abs(a) @ np.abs(b).T)


CASES = [
    (4, 512, 256, 0.0, False),        # dense layer
    (4, 512, 256, 1.0, False),        # BitLinear layer
    (5, 300, 192, 0.37, True),        # ragged tiles, gain
    (130, 260, 1024, 0.5, False),     # two token tiles and three weight tiles, both ragged
    (1, 129, 64, 0.9, True),          # one token, one K stage pair
    (64, 1024, 4096, 0.25, True),     # 7B-sized K
    (300, 128, 2048, 0.75, False),    # many token tiles
]


@pytest.mark.parametrize("M,N,K,lam,with_gain", CASES)
def test_blend_matches_oracle(orc, dev, M, N, K, lam, with_gain):
    print(f"blend case M={M} N={N} K={K} lambda={lam} gain={with_gain}", flush=True)
    x = synth.activations(M, K, 4100 + M, 4101 + M, outlier_frac=0.01, outlier_factor=20.0)
    W = synth.weights(N, K, 4102 + N)
    g = np.random.default_rng(K + N).uniform(0.5, 1.5, K).astype(np.float32) if with_gain else None
    Wd = torch.from_numpy(W).to(dev)
    packed, w_scale = bt.pack_weights(Wd)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    gd = None if g is None else torch.from_numpy(g).to(dev)
    y = bt.linear_forward_blend(xd, Wd, packed, w_scale, lam, gain=gd)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    want = orc.linear_forward_blend(x, W, lam, gain=g)
    err = np.abs(got - want)
    bound = _bound(orc, x, W, g, lam, K)
    assert (err <= bound).all(), f"max err/bound {np.max(err / bound):.3g}"
    assert np.median(err / bound) < 0.05


def test_blend_at_one_agrees_with_the_bitlinear_forward(orc, dev):
    M, N, K = 8, 1024, 4096
    x = synth.activations(M, K, 4200, 4201, outlier_frac=0.01, outlier_factor=20.0)
    W = torch.from_numpy(synth.weights(N, K, 4202)).to(dev)
    packed, w_scale = bt.pack_weights(W)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    y1 = bt.linear_forward_blend(xd, W, packed, w_scale, 1.0).cpu().numpy().astype(np.float64)
    q, dx, qs = bt.quant_act(xd)
    y = bt.linear_forward(q, dx, qs, packed, w_scale).cpu().numpy().astype(np.float64)
    # float32 sums of exact products d_x q d_w c against the exact integer sum
    assert np.allclose(y1, y, rtol=0, atol=(K + 16) * U * np.abs(y).max() + 1e-30)


def test_blend_graph_replays_match_eager(dev):
    M, N, K = 16, 256, 512
    W = torch.from_numpy(synth.weights(N, K, 4300)).to(dev)
    packed, w_scale = bt.pack_weights(W)
    xs = [torch.from_numpy(synth.activations(M, K, 4301 + i).view(np.int16)).to(dev).view(torch.bfloat16)
          for i in range(3)]
    eager = [bt.linear_forward_blend(xi, W, packed, w_scale, 0.4).cpu().clone() for xi in xs]
    x = xs[0].clone()
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    ws = torch.empty(bt.lib().bitnet_linear_forward_blend_workspace_bytes(M, K), dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            bt.linear_forward_blend(x, W, packed, w_scale, 0.4, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(6):
        x.copy_(xs[rep % 3])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.cpu(), eager[rep % 3])
