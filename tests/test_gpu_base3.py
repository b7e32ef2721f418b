"""GPU parity of the base-3 weight packing (five weights per byte) and of the
one-token GEMV that reads it, against the CPU oracle.

Bars: the repacked bytes and the int32 accumulators are bit-exact (the digits
are the same offset codes as in the 2-bit layout); outputs within 1e-5
relative.  The GEMV is fed the oracle's own base-3 packing, so its test does not
depend on the GPU repack.
"""
import numpy as np
import pytest

import bit_gemm_ternary_amd as bt
from bit_gemm_ternary_amd import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("N,K", [(1, 64), (100, 320), (37, 4160), (4096, 4096), (4096, 11008), (7, 16384),
                                 (33, 20480), (3, 65536)])
def test_pack_base3_matches_the_oracle(orc, dev, N, K):
    packed, _, _, q = orc.pack_weights(synth.weights(N, K, seed=600 + K % 97))
    rb = bt.base3_row_bytes(K)
    assert rb == -(-(-(-K // 5)) // 16) * 16
    got = host(bt.pack_base3(to_dev(packed, dev), K))
    np.testing.assert_array_equal(got, orc.pack_base3(q, rb))


# The shapes reach every batch layout of the GEMV: one to sixteen rows per
# wave in one register set, and two alternating sets at one to four chunks per
# lane (40000 x 4096, 20000 x 8192, 9000 x 12800, 5000 x 16384).
@pytest.mark.parametrize("N,K", [(1, 64), (77, 64), (1000, 320), (4096, 4096), (11008, 4096), (4096, 11008),
                                 (5000, 16384), (300, 20480), (4099, 8192), (40000, 4096), (20000, 8192),
                                 (9000, 12800), (32768, 4096)])
def test_linear_forward_base3_matches_the_oracle(orc, dev, N, K):
    W = synth.weights(N, K, seed=610 + N % 89)
    packed, d_w, _, q = orc.pack_weights(W)
    x = synth.activations(1, K, 611 + K % 53, 612, outlier_frac=0.01, outlier_factor=20.0)
    xq, d_x, qsum = orc.quant_act(x)
    want_acc, want_y = orc.linear_forward(xq, d_x, packed, d_w, K)
    p3 = orc.pack_base3(q, bt.base3_row_bytes(K))
    y, acc = bt.linear_forward_base3(to_dev(xq, dev), to_dev(d_x, dev), to_dev(qsum, dev), to_dev(p3, dev),
                                     to_dev(np.array([d_w, 0], np.float32), dev), return_acc=True)
    np.testing.assert_array_equal(host(acc), want_acc)
    got = host(y).astype(np.float64)
    assert np.all(np.abs(got - want_y) <= 1e-5 * np.abs(want_y))


def test_two_bit_and_base3_paths_agree(dev):
    # the whole chain on the GPU: pack, repack, quantise, both contractions
    N, K = 11008, 4096
    W = to_dev(synth.weights(N, K, seed=620), dev)
    packed, ws = bt.pack_weights(W)
    p3 = bt.pack_base3(packed, K)
    x = torch.from_numpy(synth.activations(1, K, 621, 622).view(np.int16)).to(dev).view(torch.bfloat16)
    q, dx, qs = bt.quant_act(x)
    y2, a2 = bt.linear_forward(q, dx, qs, packed, ws, return_acc=True)
    y3, a3 = bt.linear_forward_base3(q, dx, qs, p3, ws, return_acc=True)
    np.testing.assert_array_equal(host(a3), host(a2))
    np.testing.assert_array_equal(host(y3), host(y2))


def test_unsupported_requests_are_refused(dev):
    K = 4096
    q = torch.zeros((2, K), dtype=torch.int8, device=dev)
    s = torch.ones(2, dtype=torch.float32, device=dev)
    qs = torch.zeros(2, dtype=torch.int32, device=dev)
    p3 = torch.zeros((8, bt.base3_row_bytes(K)), dtype=torch.uint8, device=dev)
    ws = torch.ones(2, dtype=torch.float32, device=dev)
    with pytest.raises(bt.BitnetError):          # two tokens
        bt.linear_forward_base3(q, s, qs, p3, ws)
    big = 20544
    with pytest.raises(bt.BitnetError):          # K above 20480
        bt.linear_forward_base3(torch.zeros((1, big), dtype=torch.int8, device=dev), s[:1], qs[:1],
                                torch.zeros((8, bt.base3_row_bytes(big)), dtype=torch.uint8, device=dev), ws)
