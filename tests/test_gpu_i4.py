"""GPU parity of the packed 4-bit activation path (BitNet v2 summary,
"초저용량 LLM의 진화: BitNet v2 파헤치기", section 방법론: 4-bit activations).

bitnet_hadamard_quant_act_i4 must write the oracle's H-path codes packed by
the oracle's nibble encoding byte for byte, with the oracle's code sums and
scales; bitnet_linear_forward_i4 must give the oracle's int32 accumulators
bit-exactly (outputs within 1e-5 relative), on the GEMV (M <= 4) and on every
matrix-core tile configuration, at ragged sizes and at the H-BitLinear shapes.
"""
import numpy as np
import pytest

import bit_gemm_ternary_amd as bt
from bit_gemm_ternary_amd import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

RTOL = 1e-5


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


def assert_close_rel(got, want, rtol=RTOL):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    bad = np.abs(got - want) > rtol * np.abs(want)
    assert not bad.any(), (f"{bad.sum()} of {bad.size} values off by more than {rtol} relative; "
                           f"first at {np.argwhere(bad)[0]}: got {got[bad][0]} want {want[bad][0]}")


def _tokens(M, K, seed):
    return synth.activations(M, K, seed, seed + 1, dist="student_t", outlier_frac=0.0)


@pytest.mark.parametrize("M,K,with_gain", [(1, 256, False), (3, 512, True), (5, 1024, False),
                                            (7, 4096, True), (512, 4096, False), (2, 8192, True),
                                            (33, 16384, False), (2, 32768, True)])
def test_hadamard_quant_act_i4(orc, dev, M, K, with_gain):
    x = _tokens(M, K, 1700 + M)
    x[0, :] = 0                                      # an all-zero token: zero codes, zero scale
    gain = np.random.default_rng(K).uniform(0.5, 1.5, K).astype(np.float32) if with_gain else None
    wq, wdx, wqs = orc.hadamard_quant_act(x, gain=gain)
    xq4, xs, qs = bt.hadamard_quant_act_i4(bf16_to_dev(x, dev), None if gain is None else to_dev(gain, dev))
    np.testing.assert_array_equal(host(xq4), orc.pack_nibbles(wq))
    np.testing.assert_array_equal(host(qs), wqs)
    assert_close_rel(host(xs), wdx)
    assert host(xs)[0] == 0


I4_FORWARD_CASES = [
    # GEMV (M <= 4)
    (1, 100, 256), (1, 4096, 4096), (2, 1000, 4096), (3, 77, 14336), (4, 4097, 8192),
    (1, 130, 32768), (1, 40000, 4096), (1, 70000, 4096), (2, 6000, 12288), (1, 8192, 28672),
    (1, 1, 64), (4, 9, 16384),
    # matrix-core tiles, ragged M, N and K
    (5, 512, 256), (17, 1000, 4096), (100, 333, 192), (33, 65, 64),
    (2100, 14000, 192),   # 448 x 128 tiles
    (2000, 4100, 64),     # 128 x 128 tiles
    (250, 16400, 192),    # 128 x 128 tiles (few tokens, many rows)
    (999, 4100, 320),     # 128 x 128 tiles, about one round
    (300, 5000, 320),     # 128 x 64 tiles, two K groups
    (300, 4000, 320),     # 64 x 64 tiles, two K groups
    (200, 900, 4160),     # 64 x 64 tiles, four K groups, 17 stages
    (100, 333, 12352),    # 64 x 64 tiles, four K groups
]


@pytest.mark.parametrize("M,N,K", I4_FORWARD_CASES)
def test_linear_forward_i4(orc, dev, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    codes = rng.integers(-8, 8, (M, K)).astype(np.int8)
    codes[0, : K // 2] = -8                           # extreme codes
    if M > 2:
        codes[1, :] = 0                               # an all-zero token
    W = synth.weights(N, K, seed=1800 + N % 97)
    packed, d_w, _, _ = orc.pack_weights(W)
    d_x = rng.uniform(1e-3, 1e-2, M).astype(np.float32)
    qsum = codes.astype(np.int64).sum(axis=1).astype(np.int32)
    want_acc, want_y = orc.linear_forward(codes, d_x, packed, d_w, K)
    y, acc = bt.linear_forward_i4(to_dev(orc.pack_nibbles(codes), dev), to_dev(d_x, dev), to_dev(qsum, dev),
                                  to_dev(packed, dev), to_dev(np.array([d_w, 0], np.float32), dev),
                                  return_acc=True)
    acc = host(acc)
    mism = np.count_nonzero(acc != want_acc)
    assert mism == 0, f"{mism} of {acc.size} accumulators differ; first {np.argwhere(acc != want_acc)[0]}"
    assert_close_rel(host(y), want_y)


@pytest.mark.parametrize("M,N,K", [(512, 4096, 4096), (512, 4096, 16384), (1, 4096, 4096), (4, 11008, 4096)])
def test_h_bitlinear_i4_matches_int8_path(orc, dev, M, N, K):
    """Full H-BitLinear at the benchmark shapes: the packed 4-bit path gives the
    int8-container path's accumulators and outputs bit for bit, and both match
    the oracle on samples."""
    W = synth.weights(N, K, 1900)
    x_bits = _tokens(M, K, 1901)
    x = bf16_to_dev(x_bits, dev)
    packed, w_scale = bt.pack_weights(to_dev(W, dev), hadamard=True)
    xq, xs, qs = bt.hadamard_quant_act(x)
    y8, acc8 = bt.linear_forward(xq, xs, qs, packed, w_scale, return_acc=True)
    xq4, xs4, qs4 = bt.hadamard_quant_act_i4(x)
    y4, acc4 = bt.linear_forward_i4(xq4, xs4, qs4, packed, w_scale, return_acc=True)
    np.testing.assert_array_equal(host(xs4), host(xs))
    np.testing.assert_array_equal(host(acc4), host(acc8))
    np.testing.assert_array_equal(host(y4), host(y8))
    wq, _, _ = orc.hadamard_quant_act(x_bits)
    np.testing.assert_array_equal(host(xq4), orc.pack_nibbles(wq))
    rng = np.random.default_rng(5)
    rows, cols = rng.integers(0, M, 2000), rng.integers(0, N, 2000)
    want = orc.int_gemm_sampled(wq, host(packed), K, rows, cols)
    np.testing.assert_array_equal(host(acc4)[rows, cols], want)
