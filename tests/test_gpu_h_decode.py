"""GPU parity of the fused H-BitLinear forward (BitNet v2 summary,
"초저용량 LLM의 진화: BitNet v2 파헤치기", section 방법론: the layer input is
Hadamard transformed and quantised to 4-bit per-token absmax codes before the
ternary contraction).

bitnet_hadamard_bitlinear_forward must write the oracle's H-path codes packed
by the oracle's nibble encoding byte for byte, the oracle's code sums, and the
oracle's int32 accumulators bit-exactly (scales and outputs within 1e-5
relative), both where one token runs in the single fused launch (K 1024 ..
16384, every rows-per-wave count of one register set, ragged N) and where the
call runs the quantisation and contraction kernels back to back (small K,
large N, K = 32768, several tokens).
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


def fused_domain(M, N, K):
    """Shapes the single fused launch takes (the rest run two kernels)."""
    ch = max(1, K // 4096)
    waves = 2048 if K >= 8192 else 1024
    return M == 1 and 1024 <= K <= 16384 and N >= 1 and -(-N // waves) * ch <= 16


FORWARD_CASES = [
    # one fused launch: K 1024 .. 16384, rows per wave 1 .. 16
    (1, 1, 1024, False), (1, 1000, 1024, True), (1, 1025, 1024, False), (1, 16383, 1024, False),
    (1, 3000, 2048, True), (1, 4096, 4096, False), (1, 4097, 4096, True), (1, 16384, 4096, False),
    (1, 11008, 4096, False), (1, 8192, 8192, False), (1, 7001, 8192, True), (1, 16384, 8192, False),
    (1, 4096, 16384, False), (1, 3000, 16384, True), (1, 8192, 16384, False), (1, 5, 16384, False),
    # two launches: K below 1024 or 32768, N past one register set, several tokens
    (1, 100, 256, False), (1, 513, 512, True), (1, 8193, 16384, False), (1, 16385, 4096, False),
    (1, 300, 32768, False), (2, 1000, 4096, True), (4, 300, 8192, False), (9, 700, 2048, False),
]


@pytest.mark.parametrize("M,N,K,with_gain", FORWARD_CASES)
def test_hadamard_bitlinear_forward(orc, dev, M, N, K, with_gain):
    print(f"case M={M} N={N} K={K} gain={with_gain} fused={fused_domain(M, N, K)}", flush=True)
    x = synth.activations(M, K, 2100 + N % 89, 2101, dist="student_t", outlier_frac=0.0)
    gain = np.random.default_rng(K + 3).uniform(0.5, 1.5, K).astype(np.float32) if with_gain else None
    W = synth.weights(N, K, seed=2200 + N % 101)
    packed, d_w, _, _ = orc.pack_weights(W)
    wq, wdx, wqs = orc.hadamard_quant_act(x, gain=gain)
    want_acc, want_y = orc.linear_forward(wq, wdx, packed, d_w, K)
    acc_out = torch.empty((M, N), dtype=torch.int32, device=dev)
    xq4 = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    xs = torch.empty(M, dtype=torch.float32, device=dev)
    qs = torch.empty(M, dtype=torch.int32, device=dev)
    y, acc = bt.hadamard_bitlinear_forward(bf16_to_dev(x, dev), to_dev(packed, dev),
                                           to_dev(np.array([d_w, 0], np.float32), dev),
                                           gain=None if gain is None else to_dev(gain, dev),
                                           codes=(xq4, xs, qs), acc_out=acc_out)
    np.testing.assert_array_equal(host(xq4), orc.pack_nibbles(wq))
    np.testing.assert_array_equal(host(qs), wqs)
    assert_close_rel(host(xs), wdx)
    acc = host(acc)
    mism = np.count_nonzero(acc != want_acc)
    assert mism == 0, f"{mism} of {acc.size} accumulators differ; first {np.argwhere(acc != want_acc)[0]}"
    assert_close_rel(host(y), want_y)


@pytest.mark.parametrize("K", [1024, 4096, 16384])
def test_zero_token_gives_zero_codes_scale_and_outputs(orc, dev, K):
    N = 777
    packed, d_w, _, _ = orc.pack_weights(synth.weights(N, K, seed=2300))
    x = np.zeros((1, K), np.uint16)
    acc_out = torch.empty((1, N), dtype=torch.int32, device=dev)
    codes = (torch.full((1, K // 2), 0x5A, dtype=torch.uint8, device=dev),
             torch.full((1,), 7.0, dtype=torch.float32, device=dev),
             torch.full((1,), 7, dtype=torch.int32, device=dev))
    y, acc = bt.hadamard_bitlinear_forward(bf16_to_dev(x, dev), to_dev(packed, dev),
                                           to_dev(np.array([d_w, 0], np.float32), dev), codes=codes,
                                           acc_out=acc_out)
    assert not host(codes[0]).any()
    assert host(codes[1])[0] == 0 and host(codes[2])[0] == 0
    assert not host(acc).any() and not host(y).any()


@pytest.mark.parametrize("N,K", [(4096, 4096), (4096, 16384), (14336, 4096), (1024, 8192)])
def test_fused_matches_two_launches(orc, dev, N, K):
    """One token of an H-BitLinear layer (weights packed on the device with the
    row transform): the fused launch writes the two-launch path's codes, code
    sum and accumulators bit for bit, its scale and outputs within 1e-5, and
    repeated calls give identical results."""
    W = synth.weights(N, K, 2400)
    x_bits = synth.activations(1, K, 2401, 2402, dist="student_t", outlier_frac=0.001,
                                outlier_factor=20.0)
    x = bf16_to_dev(x_bits, dev)
    packed, w_scale = bt.pack_weights(to_dev(W, dev), hadamard=True)
    xq4, xs, qs = bt.hadamard_quant_act_i4(x)
    y2, acc2 = bt.linear_forward_i4(xq4, xs, qs, packed, w_scale, return_acc=True)
    outs = []
    for _ in range(2):
        codes = (torch.empty_like(xq4), torch.empty_like(xs), torch.empty_like(qs))
        acc_out = torch.empty((1, N), dtype=torch.int32, device=dev)
        y1, acc1 = bt.hadamard_bitlinear_forward(x, packed, w_scale, codes=codes, acc_out=acc_out)
        outs.append((host(codes[0]), host(codes[1]), host(codes[2]), host(acc1), host(y1)))
    for got in outs:
        np.testing.assert_array_equal(got[0], host(xq4))
        np.testing.assert_array_equal(got[2], host(qs))
        np.testing.assert_array_equal(got[3], host(acc2))
        assert_close_rel(got[1], host(xs))
        assert_close_rel(got[4], host(y2))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)
    wq, _, _ = orc.hadamard_quant_act(x_bits)
    np.testing.assert_array_equal(outs[0][0], orc.pack_nibbles(wq))


def test_n_zero_only_quantises(orc, dev):
    K = 2048
    x_bits = synth.activations(1, K, 2500, 2501, dist="student_t", outlier_frac=0.0)
    codes = (torch.empty((1, K // 2), dtype=torch.uint8, device=dev),
             torch.empty(1, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.int32, device=dev))
    packed = torch.empty((0, K // 4), dtype=torch.uint8, device=dev)
    w_scale = torch.ones(2, dtype=torch.float32, device=dev)
    y = bt.hadamard_bitlinear_forward(bf16_to_dev(x_bits, dev), packed, w_scale, codes=codes)
    assert tuple(y.shape) == (1, 0)
    wq, wdx, wqs = orc.hadamard_quant_act(x_bits)
    np.testing.assert_array_equal(host(codes[0]), orc.pack_nibbles(wq))
    np.testing.assert_array_equal(host(codes[2]), wqs)
    assert_close_rel(host(codes[1]), wdx)


def _bf16_bits(values, K):
    x = np.zeros((1, K), np.float32)
    for i, v in values.items():
        x[0, i] = v
    return (x.view(np.uint32) >> 16).astype(np.uint16)   # every value here is exact in bf16


@pytest.mark.parametrize("K", [1024, 16384])
@pytest.mark.parametrize("a,b,half_code", [(7.5, 6.5, 0), (8.5, 5.5, 2)])
def test_rounding_ties_go_to_even(orc, dev, K, a, b, half_code):
    """x = a e_0 + b e_1 transforms to a + b and a - b; with absmax a + b = 14
    the scale is exactly 1/2, so a - b lands on a half-integer code (0.5 or
    1.5) that rounds to the even neighbour, as in the oracle."""
    N = 300
    x = _bf16_bits({0: a, 1: b}, K)
    packed, d_w, _, _ = orc.pack_weights(synth.weights(N, K, seed=2600))
    wq, wdx, wqs = orc.hadamard_quant_act(x)
    assert set(np.unique(wq)) == {7, half_code}
    want_acc, want_y = orc.linear_forward(wq, wdx, packed, d_w, K)
    codes = (torch.empty((1, K // 2), dtype=torch.uint8, device=dev),
             torch.empty(1, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.int32, device=dev))
    y, acc = bt.hadamard_bitlinear_forward(bf16_to_dev(x, dev), to_dev(packed, dev),
                                           to_dev(np.array([d_w, 0], np.float32), dev), codes=codes,
                                           acc_out=torch.empty((1, N), dtype=torch.int32, device=dev))
    np.testing.assert_array_equal(host(codes[0]), orc.pack_nibbles(wq))
    np.testing.assert_array_equal(host(codes[2]), wqs)
    assert_close_rel(host(codes[1]), wdx)
    np.testing.assert_array_equal(host(acc), want_acc)
    assert_close_rel(host(y), want_y)


@pytest.mark.parametrize("eps", [0.0, 0.25])
def test_eps_only_scales(orc, dev, eps):
    K, N = 4096, 2000
    x = synth.activations(1, K, 2700, 2701, dist="student_t", outlier_frac=0.0)
    gain = np.random.default_rng(2702).uniform(0.5, 1.5, K).astype(np.float32)
    packed, d_w, _, _ = orc.pack_weights(synth.weights(N, K, seed=2703))
    wq, wdx, wqs = orc.hadamard_quant_act(x, gain=gain, eps=eps)
    want_acc, want_y = orc.linear_forward(wq, wdx, packed, d_w, K)
    codes = (torch.empty((1, K // 2), dtype=torch.uint8, device=dev),
             torch.empty(1, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.int32, device=dev))
    y, acc = bt.hadamard_bitlinear_forward(bf16_to_dev(x, dev), to_dev(packed, dev),
                                           to_dev(np.array([d_w, 0], np.float32), dev),
                                           gain=to_dev(gain, dev), eps=eps, codes=codes,
                                           acc_out=torch.empty((1, N), dtype=torch.int32, device=dev))
    np.testing.assert_array_equal(host(codes[0]), orc.pack_nibbles(wq))
    assert_close_rel(host(codes[1]), wdx)
    np.testing.assert_array_equal(host(acc), want_acc)
    assert_close_rel(host(y), want_y)
